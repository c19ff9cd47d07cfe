// Step 2 of the ThriftAttention path ("ThriftAttention: Selective Mixed
// Precision for Long-Context FP4 Attention", abstract: a fast heuristic marks
// the few important query-key block pairs that stay in FP16).
//
// Heuristic: mean-pool every 64-row block of Q (per query head) and K (per
// KV head); score the pair (i, j) by the fp64 dot product of the means taken
// in channel order; per (b, h_q, i) keep the first and diagonal key blocks
// and the best-scoring others up to ceil(frac * valid blocks) in total.
//
// Three kernels:
//   pool_kernel     the pooled means (exact fp64 sums, one rounding to fp32);
//   score_kernel    every causal block score of a 64 x 64 tile of (query
//                   block, key block) pairs per workgroup, from pooled means
//                   staged once in LDS; the scores, rounded to fp32, go into
//                   the list array at the positions the lists will occupy;
//   select_kernel   one wave per query-block row: the cut-off among the row's
//                   fp32 scores by a bitwise search, an exact fp64 decision
//                   for the blocks tied with it, then both lists in place.
//
// Bit-exactness: the pooled sums of 64 fp16 values are exact in fp64 (they
// need at most 46 significant bits), so their order does not matter; each
// product of two fp32 means is exact in fp64, so a sequential fma chain in
// channel order gives the same bits as any sequential multiply-add in that
// order.  Rounding a score to fp32 keeps the order of unequal fp32 values
// (the rounding is monotone), so only blocks whose fp32 score equals the
// cut-off need their fp64 scores, which the select kernel recomputes with
// the same chain.
#include <mutex>

#include "thrift_internal.h"

namespace thrift {

// One thread per (head row-block, channel).  Q means are written row-major
// [BH, nb, d]; K means transposed [BH, d, nb] so that the scoring kernel
// stages them coalesced.
template <bool TRANSPOSED>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t *__restrict__ x16, float *__restrict__ out,
                                                   int64_t BH, int N, int d) {
  const int nb = N / 64;
  const int64_t total = BH * nb * d;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(t % d);
    const int64_t bi = t / d;  // = bh * nb + i
    const int64_t bh = bi / nb;
    const int i = (int)(bi % nb);
    const uint16_t *p = x16 + (bh * N + 64 * (int64_t)i) * d + c;
    double s = 0.0;
#pragma unroll 8
    for (int r = 0; r < 64; r++) s += (double)__builtin_bit_cast(_Float16, p[(int64_t)r * d]);
    const float m = (float)(s * (1.0 / 64.0));
    if (TRANSPOSED)
      out[(bh * d + c) * nb + i] = m;
    else
      out[bi * d + c] = m;
  }
}

// Causal rows start at i(i+1)/2 and hold i + 1 entries; others at i nb.
__device__ __forceinline__ int64_t row_offset(const int i, const int nb, const int causal) {
  return causal ? (int64_t)i * (i + 1) / 2 : (int64_t)i * nb;
}

// ---------------------------------------------------------------------------
// Scoring.  One workgroup (256 threads) per (b, h_q, tile of 64 query blocks
// x 64 key blocks); causal heads take the tiles on and below the diagonal.
// The tile's pooled means are staged in LDS as fp64, channel-major, 64
// channels at a time (two workgroups fit on a CU, so one stages while the
// other computes); thread t owns query blocks 4 (t / 16) + 0..3 and key
// blocks 4 (t % 16) + 0..3 and runs their 16 fma chains over the channels
// in order.
constexpr int kScoreThreads = 256;
constexpr int kChunk = 64;    // channels staged at a time
constexpr int kQStride = 66;  // doubles per channel row of the staged Q tile (16-byte aligned, fewer bank conflicts)
constexpr int kScoreLds = kChunk * (kQStride + 64) * 8;

template <int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(SelectArgs a, int tiles_per_head, int tn) {
  extern __shared__ __attribute__((aligned(16))) double sm[];
  double *qs = sm, *ks = sm + kChunk * kQStride;
  const int nb = a.N / 64;
  const int64_t bh = blockIdx.x / tiles_per_head;
  const int t = blockIdx.x % tiles_per_head;
  int ti, tj;
  if (a.causal) {
    ti = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= t) ti++;
    while (ti * (ti + 1) / 2 > t) ti--;
    tj = t - ti * (ti + 1) / 2;
  } else {
    ti = t / tn;
    tj = t % tn;
  }
  const int i0 = 64 * ti, j0 = 64 * tj;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = (int)((int64_t)h * a.Hkv / a.Hq);
  const int tid = threadIdx.x;
  const float *qb = a.qbar + (bh * nb + i0) * (int64_t)D;                     // Q means, row-major
  const float *kb = a.kbarT + ((int64_t)b * a.Hkv + g) * D * (int64_t)nb + j0;  // K means, channel-major
  const int qi = 4 * (tid >> 4), kj = 4 * (tid & 15);
  double s[4][4];
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int v = 0; v < 4; v++) s[u][v] = 0.0;
  for (int c0 = 0; c0 < D; c0 += kChunk) {
    // every staging load is issued before any is used: 4 float4 of Q
    // (row r, channels c0 + 4 q4 ..) and 16 floats of K (channel c, blocks
    // j0 + 4 jq ..) per thread; blocks past nb read as 0
    float4 qv[4];
    float kv[4][4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int e = tid + kScoreThreads * u, r = e >> 4, q4 = e & 15;
      const int rr = min(r, nb - 1 - i0);  // in bounds; rows past nb are zeroed below
      qv[u] = *(const float4 *)(qb + (int64_t)rr * D + c0 + 4 * q4);
      const int c = e >> 4, jq = e & 15;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int jj = min(4 * jq + v, nb - 1 - j0);
        kv[u][v] = kb[(int64_t)(c0 + c) * nb + jj];
      }
    }
    if (c0 > 0) __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int e = tid + kScoreThreads * u, r = e >> 4, q4 = e & 15;
      const bool rok = i0 + r < nb;
      qs[(4 * q4 + 0) * kQStride + r] = rok ? (double)qv[u].x : 0.0;
      qs[(4 * q4 + 1) * kQStride + r] = rok ? (double)qv[u].y : 0.0;
      qs[(4 * q4 + 2) * kQStride + r] = rok ? (double)qv[u].z : 0.0;
      qs[(4 * q4 + 3) * kQStride + r] = rok ? (double)qv[u].w : 0.0;
      const int c = e >> 4, jq = e & 15;
#pragma unroll
      for (int v = 0; v < 4; v++) ks[c * 64 + 4 * jq + v] = (j0 + 4 * jq + v < nb) ? (double)kv[u][v] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kChunk; c++) {
      const double2 q01 = *(const double2 *)(qs + c * kQStride + qi);
      const double2 q23 = *(const double2 *)(qs + c * kQStride + qi + 2);
      const double2 k01 = *(const double2 *)(ks + c * 64 + kj);
      const double2 k23 = *(const double2 *)(ks + c * 64 + kj + 2);
      const double qd[4] = {q01.x, q01.y, q23.x, q23.y}, kd[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int v = 0; v < 4; v++) s[u][v] = fma(qd[u], kd[v], s[u][v]);
    }
  }
  // the fp32 roundings of the scores, at the list positions of the rows
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  int32_t *base = a.idx + bh * per;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int i = i0 + qi + u;
    if (i >= nb) continue;
    const int nv = a.causal ? i + 1 : nb;
    int32_t *row = base + row_offset(i, nb, a.causal);
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int j = j0 + kj + v;
      if (j < nv) row[j] = __float_as_int((float)s[u][v]);
    }
  }
}

// Tile (ti, tj) of head-tile index t (causal heads: the tiles on and below the diagonal,
// row-major; else tn x tn).
__device__ __forceinline__ void tile_of(const int t, const int causal, const int tn, int &ti, int &tj) {
  if (causal) {
    ti = (int)((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= t) ti++;
    while (ti * (ti + 1) / 2 > t) ti--;
    tj = t - ti * (ti + 1) / 2;
  } else {
    ti = t / tn;
    tj = t % tn;
  }
}

// ---------------------------------------------------------------------------
// The selection's own scoring of pooled means, in fp32.  The selection
// needs the order of the fp64 chains, not their values: a sequential fp32
// fma chain over d channels differs from the exact dot product by at most
// gamma_d sum_c |q_c k_c| <= gamma_d |q| |k| (gamma_d = d u / (1 - d u),
// u = 2^-24; Cauchy-Schwarz), and the fp64 chain from it by far less, so
// every fp32 score lies within M = 2 d 2^-24 |q_i| max_j |k_j| of the fp64
// score (the factor 2 covers gamma_d's own correction, the fp64 chain's
// error and the norms' roundings, all below 2^-40 relative).  The select
// kernel takes every block whose fp32 score clears the fp32 cut-off by more
// than 2M, drops every block below it by more than 2M, and decides the rest
// by their fp64 chains: the same lists as ranking every fp64 score.

// Euclidean norms of the Q means ([BH, nb], row-major source): fp64 sum of
// the exact squares, fp64 sqrt, rounded up to fp32.  One thread per row.
template <int D>
__global__ __launch_bounds__(256) void qnorm_kernel(const float *__restrict__ qbar, float *__restrict__ qn,
                                                    const int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const float4 *q = (const float4 *)(qbar + r * D);
  double ss = 0.0;
#pragma unroll 8
  for (int c = 0; c < D / 4; c++) {
    const float4 v = q[c];
    ss = fma((double)v.x, (double)v.x, ss);
    ss = fma((double)v.y, (double)v.y, ss);
    ss = fma((double)v.z, (double)v.z, ss);
    ss = fma((double)v.w, (double)v.w, ss);
  }
  qn[r] = __double2float_ru(sqrt(ss));
}

// Norms of the K means ([BHkv, d, nb], channel-major source): one thread
// per block, so consecutive threads read consecutive blocks of a channel.
template <int D>
__global__ __launch_bounds__(256) void knorm_kernel(const float *__restrict__ kbarT, float *__restrict__ kn,
                                                    const int nb, const int64_t blocks) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // = hk * nb + j
  if (e >= blocks) return;
  const int64_t hk = e / nb;
  const int j = (int)(e % nb);
  const float *kb = kbarT + hk * D * (int64_t)nb + j;
  double ss = 0.0;
#pragma unroll 8
  for (int c = 0; c < D; c++) {
    const double v = (double)kb[(int64_t)c * nb];
    ss = fma(v, v, ss);
  }
  kn[e] = __double2float_ru(sqrt(ss));
}

// Per KV head, the largest K-mean norm over blocks 1 .. nb-1 (block 0 is
// always on the FP16 list, never a candidate).  One workgroup per KV head.
__global__ __launch_bounds__(256) void knmax_kernel(const float *__restrict__ kn, float *__restrict__ knmax,
                                                    const int nb) {
  __shared__ float part[4];
  const int64_t hk = blockIdx.x;
  float mx = 0.0f;
  for (int j = 1 + threadIdx.x; j < nb; j += 256) mx = fmaxf(mx, kn[hk * nb + j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) knmax[hk] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

// fp32 pooled-mean scores: every causal score of a 128 x 128 tile of (query
// block, key block) pairs per workgroup of 256 threads, written as fp32 bits
// at the list positions.  Thread (tr, tc) = (t / 16, t % 16) owns query
// blocks 4 tr + {0..3, 64..67} and key blocks 4 tc + {0..3, 64..67}, so each
// channel step reads 4 x 16 bytes of LDS (consecutive lanes, consecutive
// 16-byte chunks) for 64 fmas; the means are staged 32 channels at a time,
// channel-major, and each chain runs over the channels in order.
constexpr int kS32Tile = 128, kS32Chunk = 32;

template <int D>
__global__ __launch_bounds__(256) void score32_kernel(SelectArgs a, int tiles_per_head, int tn) {
  __shared__ __attribute__((aligned(16))) float qs[kS32Chunk][kS32Tile];
  __shared__ __attribute__((aligned(16))) float ks[kS32Chunk][kS32Tile];
  const int nb = a.N / 64;
  const int64_t bh = blockIdx.x / tiles_per_head;
  int ti, tj;
  tile_of(blockIdx.x % tiles_per_head, a.causal, tn, ti, tj);
  const int i0 = kS32Tile * ti, j0 = kS32Tile * tj;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = (int)((int64_t)h * a.Hkv / a.Hq);
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const float *qb = a.qbar + (bh * nb + i0) * (int64_t)D;
  const float *kb = a.kbarT + ((int64_t)b * a.Hkv + g) * D * (int64_t)nb + j0;
  float s[8][8];
#pragma unroll
  for (int u = 0; u < 8; u++)
#pragma unroll
    for (int v = 0; v < 8; v++) s[u][v] = 0.0f;
  for (int c0 = 0; c0 < D; c0 += kS32Chunk) {
    // staging loads, all issued before any is used: Q rows (8 float4 per
    // 32-channel row segment), K channel rows (scalar: nb need not be a
    // multiple of 4); rows and blocks past nb read in bounds and become 0
    float4 qv[4];
    float kv[16];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int e = tid + 256 * u, r = e >> 3, q4 = e & 7;
      qv[u] = *(const float4 *)(qb + (int64_t)min(r, nb - 1 - i0) * D + c0 + 4 * q4);
    }
#pragma unroll
    for (int u = 0; u < 16; u++) {
      const int e = tid + 256 * u, c = e >> 7, j = e & 127;
      kv[u] = kb[(int64_t)(c0 + c) * nb + min(j, nb - 1 - j0)];
    }
    if (c0 > 0) __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int e = tid + 256 * u, r = e >> 3, q4 = e & 7;
      const bool ok = i0 + r < nb;
      qs[4 * q4 + 0][r] = ok ? qv[u].x : 0.0f;
      qs[4 * q4 + 1][r] = ok ? qv[u].y : 0.0f;
      qs[4 * q4 + 2][r] = ok ? qv[u].z : 0.0f;
      qs[4 * q4 + 3][r] = ok ? qv[u].w : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 16; u++) {
      const int e = tid + 256 * u, c = e >> 7, j = e & 127;
      ks[c][j] = (j0 + j < nb) ? kv[u] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kS32Chunk; c++) {
      const float4 qa = *(const float4 *)&qs[c][4 * tr], qb4 = *(const float4 *)&qs[c][64 + 4 * tr];
      const float4 ka = *(const float4 *)&ks[c][4 * tc], kb4 = *(const float4 *)&ks[c][64 + 4 * tc];
      const float qd[8] = {qa.x, qa.y, qa.z, qa.w, qb4.x, qb4.y, qb4.z, qb4.w};
      const float kd[8] = {ka.x, ka.y, ka.z, ka.w, kb4.x, kb4.y, kb4.z, kb4.w};
#pragma unroll
      for (int u = 0; u < 8; u++)
#pragma unroll
        for (int v = 0; v < 8; v++) s[u][v] = fmaf(qd[u], kd[v], s[u][v]);
    }
  }
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  int32_t *base = a.idx + bh * per;
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int i = i0 + 4 * tr + (u & 3) + 64 * (u >> 2);
    if (i >= nb) continue;
    const int nv = a.causal ? i + 1 : nb;
    int32_t *row = base + row_offset(i, nb, a.causal);
#pragma unroll
    for (int v = 0; v < 8; v++) {
      const int j = j0 + 4 * tc + (v & 3) + 64 * (v >> 2);
      if (j < nv) row[j] = __float_as_int(s[u][v]);
    }
  }
}

// ---------------------------------------------------------------------------
// Other block scores (the heuristic is the method's open risk: the
// hotpaper.ai summary of the ThriftAttention paper, section on significance
// and limits).  Each replaces the pooled mean; the selection is unchanged.
// All chains are fp64 in the order stated, as in the pooled score.
enum { kScorePooled = 0, kScoreMaxPooled = 1, kScoreNormWeighted = 2, kScoreBlockMax = 3 };

__device__ __forceinline__ double half_to_double(const uint16_t h) { return (double)__builtin_bit_cast(_Float16, h); }

// Norm-weighted mean of one 64-row block per workgroup: row r weighs its L2
// norm w_r (sqrt of the fma chain of squares over the channels in order);
// mean_c = (fma chain of w_r x_rc over the rows in order) / (sum of w_r in
// row order), rounded once to fp32, 0 for an all-zero block.  Q means go
// row-major [BH, nb, d], K means channel-major [BH, d, nb], as pool_kernel.
template <bool TRANSPOSED>
__global__ __launch_bounds__(128) void normw_pool_kernel(const uint16_t *__restrict__ x16, float *__restrict__ out,
                                                         int N, int d) {
  __shared__ double w[64];
  __shared__ double wsum;
  const int nb = N / 64;
  const int64_t bi = blockIdx.x;  // = bh * nb + i
  const int64_t bh = bi / nb;
  const int i = (int)(bi % nb);
  const uint16_t *blk = x16 + (bh * N + 64 * (int64_t)i) * d;
  const int tid = threadIdx.x;
  if (tid < 64) {
    double ss = 0.0;
    for (int c = 0; c < d; c++) {
      const double x = half_to_double(blk[(int64_t)tid * d + c]);
      ss = fma(x, x, ss);
    }
    w[tid] = sqrt(ss);
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int r = 0; r < 64; r++) s += w[r];
    wsum = s;
  }
  __syncthreads();
  for (int c = tid; c < d; c += 128) {
    double acc = 0.0;
    for (int r = 0; r < 64; r++) acc = fma(w[r], half_to_double(blk[(int64_t)r * d + c]), acc);
    const float m = wsum > 0.0 ? (float)(acc / wsum) : 0.0f;
    if (TRANSPOSED)
      out[(bh * d + c) * nb + i] = m;
    else
      out[bi * d + c] = m;
  }
}


// Max-pooled scores: the 64 x 64 block-pair tile of score_kernel, with the
// key side one row r of every key block at a time: the query means stay in
// LDS (fp64, channel-major) while the 64 key rows r of the tile's blocks are
// staged for each r; thread t keeps the running max of its 16 chains.
template <int D>
__global__ __launch_bounds__(kScoreThreads) void maxpool_score_kernel(SelectArgs a, int tiles_per_head, int tn) {
  extern __shared__ __attribute__((aligned(16))) double sm[];
  double *qs = sm, *ks = sm + D * kQStride;
  const int nb = a.N / 64;
  const int64_t bh = blockIdx.x / tiles_per_head;
  int ti, tj;
  tile_of(blockIdx.x % tiles_per_head, a.causal, tn, ti, tj);
  const int i0 = 64 * ti, j0 = 64 * tj;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = (int)((int64_t)h * a.Hkv / a.Hq);
  const int tid = threadIdx.x;
  const float *qb = a.qbar + (bh * nb + i0) * (int64_t)D;
  for (int e = tid; e < 64 * D; e += kScoreThreads) {
    const int r = e / D, c = e % D;
    qs[c * kQStride + r] = (i0 + r < nb) ? (double)qb[(int64_t)min(r, nb - 1 - i0) * D + c] : 0.0;
  }
  const uint16_t *kh = a.k16 + ((int64_t)b * a.Hkv + g) * a.N * (int64_t)D;
  const int qi = 4 * (tid >> 4), kj = 4 * (tid & 15);
  double best[4][4];
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int v = 0; v < 4; v++) best[u][v] = -INFINITY;
  for (int r = 0; r < 64; r++) {
    __syncthreads();  // the previous row's reads are done (and the Q tile is staged)
    for (int e = tid; e < 64 * D; e += kScoreThreads) {
      const int jj = e / D, c = e % D;
      const int j = min(j0 + jj, nb - 1);  // in bounds; blocks past nb are never written
      ks[c * 64 + jj] = half_to_double(kh[((int64_t)64 * j + r) * D + c]);
    }
    __syncthreads();
    double s[4][4];
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int v = 0; v < 4; v++) s[u][v] = 0.0;
#pragma unroll 4
    for (int c = 0; c < D; c++) {
      const double2 q01 = *(const double2 *)(qs + c * kQStride + qi);
      const double2 q23 = *(const double2 *)(qs + c * kQStride + qi + 2);
      const double2 k01 = *(const double2 *)(ks + c * 64 + kj);
      const double2 k23 = *(const double2 *)(ks + c * 64 + kj + 2);
      const double qd[4] = {q01.x, q01.y, q23.x, q23.y}, kd[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int v = 0; v < 4; v++) s[u][v] = fma(qd[u], kd[v], s[u][v]);
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int v = 0; v < 4; v++) best[u][v] = fmax(best[u][v], s[u][v]);
  }
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  int32_t *base = a.idx + bh * per;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int i = i0 + qi + u;
    if (i >= nb) continue;
    const int nv = a.causal ? i + 1 : nb;
    int32_t *row = base + row_offset(i, nb, a.causal);
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int j = j0 + kj + v;
      if (j < nv) row[j] = __float_as_int((float)best[u][v]);
    }
  }
}

// Block-max scores: a workgroup per valid (b, h_q, i, j) at a time (grid
// stride: B Hq times the valid pairs can exceed what one launch addresses):
// both blocks' 64 rows staged in LDS (fp64, channel-major), thread t runs 16
// of the 4096 row-pair chains, and the workgroup takes the max.
template <int D>
__device__ void blockmax_pair(const SelectArgs &a, const int64_t per, const int64_t bh, const int64_t p) {
  extern __shared__ __attribute__((aligned(16))) double sm[];
  __shared__ double wmax[kScoreThreads / 64];
  double *qs = sm, *ks = sm + D * kQStride;
  const int nb = a.N / 64;
  int i, j;
  if (a.causal) {
    i = (int)((sqrt(8.0 * (double)p + 1.0) - 1.0) * 0.5);
    while ((int64_t)(i + 1) * (i + 2) / 2 <= p) i++;
    while ((int64_t)i * (i + 1) / 2 > p) i--;
    j = (int)(p - (int64_t)i * (i + 1) / 2);
  } else {
    i = (int)(p / nb);
    j = (int)(p % nb);
  }
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = (int)((int64_t)h * a.Hkv / a.Hq);
  const uint16_t *qblk = a.q16 + (bh * a.N + 64 * (int64_t)i) * D;
  const uint16_t *kblk = a.k16 + (((int64_t)b * a.Hkv + g) * a.N + 64 * (int64_t)j) * D;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * D; e += kScoreThreads) {
    const int r = e / D, c = e % D;
    qs[c * kQStride + r] = half_to_double(qblk[e]);
    ks[c * 64 + r] = half_to_double(kblk[e]);
  }
  __syncthreads();
  const int qi = 4 * (tid >> 4), kj = 4 * (tid & 15);
  double s[4][4];
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int v = 0; v < 4; v++) s[u][v] = 0.0;
#pragma unroll 4
  for (int c = 0; c < D; c++) {
    const double2 q01 = *(const double2 *)(qs + c * kQStride + qi);
    const double2 q23 = *(const double2 *)(qs + c * kQStride + qi + 2);
    const double2 k01 = *(const double2 *)(ks + c * 64 + kj);
    const double2 k23 = *(const double2 *)(ks + c * 64 + kj + 2);
    const double qd[4] = {q01.x, q01.y, q23.x, q23.y}, kd[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int v = 0; v < 4; v++) s[u][v] = fma(qd[u], kd[v], s[u][v]);
  }
  double m = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int v = 0; v < 4; v++) m = fmax(m, s[u][v]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    double best = wmax[0];
    for (int w = 1; w < kScoreThreads / 64; w++) best = fmax(best, wmax[w]);
    const int64_t tri = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
    a.idx[bh * tri + row_offset(i, nb, a.causal) + j] = __float_as_int((float)best);
  }
  __syncthreads();  // the next pair restages qs/ks and wmax
}

template <int D>
__global__ __launch_bounds__(kScoreThreads) void blockmax_score_kernel(SelectArgs a, int64_t per) {
  const int64_t total = (int64_t)a.B * a.Hq * per;
  for (int64_t w = blockIdx.x; w < total; w += gridDim.x) blockmax_pair<D>(a, per, w / per, w % per);
}

// ---------------------------------------------------------------------------
// Selection: one wave per (b, h_q, query block i).
constexpr int kSelThreads = 256;

// Order-preserving maps to unsigned keys (larger value -> larger key), with
// -0 folded onto +0 so that equal scores compare equal.  Every finite value
// maps above 0, which marks "not a candidate".
__device__ __forceinline__ uint32_t order_key32_bits(uint32_t u) {
  u = (u << 1) ? u : 0u;  // -0 -> +0
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u; else u | sign bit
}
__device__ __forceinline__ uint64_t order_key64(double s) {
  if (s == 0.0) s = 0.0;
  const uint64_t u = __double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
// The fp32 value of a nonzero order key.
__device__ __forceinline__ float key32_value(const uint32_t k) {
  return __uint_as_float((k >> 31) ? (k & 0x7fffffffu) : ~k);
}

// Number of the wave's keys (KPL per lane) at or above c.
template <int KPL>
__device__ __forceinline__ int count_at_least(const uint32_t (&key)[KPL], const uint32_t c) {
  int n = 0;
#pragma unroll
  for (int t = 0; t < KPL; t++) n += __popcll(__ballot(key[t] >= c));
  return n;
}

// Largest value T with at least k of the wave's keys >= T, i.e. the k-th
// largest key (1 <= k <= number of nonzero keys).  Bits above the highest
// one in which the largest and the smallest nonzero key differ are common to
// every candidate, so the search starts below them; it stops as soon as
// exactly k keys lie at or above the candidate, whose smallest is then T.
template <int KPL>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[KPL], const int k) {
  uint32_t mx = 0, mn = 0xffffffffu;
#pragma unroll
  for (int t = 0; t < KPL; t++) {
    mx = max(mx, key[t]);
    mn = key[t] ? min(mn, key[t]) : mn;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
  }
  mx = __builtin_amdgcn_readfirstlane(mx);
  mn = __builtin_amdgcn_readfirstlane(mn);
  const uint32_t diff = mx ^ mn;
  if (diff == 0) return mx;
  const int top = 31 - __builtin_clz(diff);  // highest differing bit
  uint32_t t = mx & ~((top == 31) ? 0xffffffffu : ((2u << top) - 1u));
  for (int bit = top; bit >= 0; bit--) {
    const uint32_t c = t | (1u << bit);
    const int n = count_at_least<KPL>(key, c);
    if (n >= k) {
      t = c;
      if (n == k) {  // T = the smallest of those k keys
        uint32_t m = 0xffffffffu;
#pragma unroll
        for (int u = 0; u < KPL; u++) m = key[u] >= c ? min(m, key[u]) : m;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, off, 64));
        return __builtin_amdgcn_readfirstlane(m);
      }
    }
  }
  return t;
}

// The fp64 score of (query mean row qrow, key block j), the same chain as
// score_kernel: fma over the channels in order, starting from 0.
template <int D>
__device__ __forceinline__ double exact_score(const float *qrow, const float *kT, const int nb, const int j) {
  double s = 0.0;
#pragma unroll 8
  for (int c = 0; c < D; c++) s = fma((double)qrow[c], (double)kT[(int64_t)c * nb + j], s);
  return s;
}

// The fp64 block score of kind `kind` for key block j of a query row: the
// pooled or norm-weighted means' chain (qrow, kT), the max over the key rows
// of (qrow . k_r), or the max over every row pair of the two blocks.
// (A call, not inlined: the selection reaches it only for the few blocks
// near its cut-off, from several unrolled sites.)
template <int D>
__device__ __noinline__ double exact_score_kind(const int kind, const float *qrow, const float *kT, const int nb,
                                                const uint16_t *qblk, const uint16_t *kh, const int j) {
  if (kind == kScoreMaxPooled || kind == kScoreBlockMax) {
    const uint16_t *kblk = kh + (int64_t)64 * j * D;
    double best = -INFINITY;
    const int na = kind == kScoreBlockMax ? 64 : 1;
    for (int q = 0; q < na; q++)
      for (int r = 0; r < 64; r++) {
        double s = 0.0;
        for (int c = 0; c < D; c++) {
          const double qv = kind == kScoreBlockMax ? half_to_double(qblk[q * D + c]) : (double)qrow[c];
          s = fma(qv, half_to_double(kblk[r * D + c]), s);
        }
        best = fmax(best, s);
      }
    return best;
  }
  return exact_score<D>(qrow, kT, nb, j);
}

// Undecided blocks of a row (those in the band around the cut-off) are
// ranked through LDS when there are at most kBand of them: per wave kBand
// 64-bit exact keys, kBand block indices and one decision byte per block.
constexpr int kBand = 64;
__host__ __device__ constexpr size_t select_lds_per_wave(const int nb) {
  return (size_t)kBand * (8 + 4) + (((size_t)nb + 15) & ~(size_t)15);
}

// KPL: keys per lane, at least ceil(nb / 64).  Lane l holds blocks l + 64 t.
// The scores in the list array are fp32: the rounded fp64 scores of a.kind
// (margin 0: only blocks equal to the cut-off are undecided), or, for
// pooled means, the fp32 chains of score32_kernel (margin M: the blocks
// within 2M of the cut-off are undecided).  Undecided blocks are ranked by
// their fp64 scores, the lower block index first among equal ones.
template <int D, int KPL>
__global__ __launch_bounds__(kSelThreads)
__attribute__((amdgpu_waves_per_eu(KPL <= 16 ? 4 : (KPL <= 32 ? 3 : 1)))) void select_kernel(SelectArgs a,
                                                                                                const int i_lo,
                                                                                                const int i_span) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sel_lds[];
  const int nb = a.N / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // this launch's rows: query blocks [i_lo, i_lo + i_span) of every (b, h)
  const int64_t r = (int64_t)blockIdx.x * (kSelThreads / 64) + wave;
  if (r >= (int64_t)a.B * a.Hq * i_span) return;
  const int64_t bh = r / i_span;
  const int i = i_lo + (int)(r % i_span);
  const int64_t row = bh * nb + i;  // = (b*Hq + h)*nb + i
  const int nv = a.causal ? i + 1 : nb;
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  int32_t *out = a.idx + bh * per + row_offset(i, nb, a.causal);
  uint8_t *wl = sel_lds + (size_t)wave * select_lds_per_wave(nb);
  uint64_t *band_key = (uint64_t *)wl;
  int32_t *band_blk = (int32_t *)(wl + kBand * 8);
  uint8_t *decided = wl + kBand * 12;

  if (a.ppm == 0) {  // no FP16 blocks: the FP4 list is every valid block
    for (int j = lane; j < nv; j += 64) out[j] = j;
    if (lane == 0) a.n16[row] = 0;
    return;
  }
  const int nforced = (i == 0) ? 1 : 2;
  int64_t want = (a.ppm * nv + 999999) / 1000000;
  int64_t kk = want > nforced ? want : nforced;
  if (kk > nv) kk = nv;
  const int kextra = (int)kk - nforced;  // best non-forced blocks to add
  const bool scored = kextra > 0 && kextra < nv - nforced;

  // key: order key of the block's fp32 score (0: not a candidate).  Blocks
  // above the band [Tlo, Thi] around the cut-off are taken; `take` of the
  // band's `nband` blocks join them: all of them (mode 0), those marked in
  // `decided` (mode 1, at most kBand in the band), or by the T64 rule (mode
  // 2, a wider band).
  uint32_t key[KPL];
  uint32_t Tlo = 0, Thi = 0;
  int mode = 0;
  uint64_t T64 = 0;
  int take_eq64 = 0;
  const float *qrow = nullptr, *kT = nullptr;
  const uint16_t *kh = nullptr, *qblk = nullptr;
  if (scored) {
    // every load is issued before any is used (an out-of-row lane reads
    // entry 0 and discards it)
    int32_t raw[KPL];
#pragma unroll
    for (int t = 0; t < KPL; t++) {
      const int j = lane + 64 * t;
      raw[t] = out[j < nv ? j : 0];
    }
#pragma unroll
    for (int t = 0; t < KPL; t++) {
      const int j = lane + 64 * t;
      const uint32_t k32 = order_key32_bits((uint32_t)raw[t]);
      key[t] = (j < nv && j != 0 && j != i) ? k32 : 0u;
    }
    const uint32_t T = kth_largest<KPL>(key, kextra);
    Tlo = Thi = T;
    const int g = (int)((int64_t)(bh % a.Hq) * a.Hkv / a.Hq), b = (int)(bh / a.Hq);
    if (a.kind == kScorePooled) {
      // fp32 chains: the band is the cut-off +- 2M, rounded outwards
      const double M = 2.0 * D * 0x1p-24 * (double)a.qn[row] * (double)a.knmax[(int64_t)b * a.Hkv + g];
      const double c = (double)key32_value(T);
      Thi = order_key32_bits(__float_as_uint(__double2float_ru(c + 2.0 * M)));
      Tlo = max(order_key32_bits(__float_as_uint(__double2float_rd(c - 2.0 * M))), 1u);
    }
    int gt = 0, nband = 0;
#pragma unroll
    for (int t = 0; t < KPL; t++) {
      gt += __popcll(__ballot(key[t] > Thi));
      nband += __popcll(__ballot(key[t] >= Tlo && key[t] <= Thi));
    }
    const int take = kextra - gt;  // 1 .. nband
    if (take < nband) {
      // the fp64 scores of the band's blocks decide; among equal fp64
      // scores the lower block index wins
      qrow = a.qbar + row * (int64_t)D;
      kT = a.kbarT + ((int64_t)b * a.Hkv + g) * D * (int64_t)nb;
      kh = a.k16 + ((int64_t)b * a.Hkv + g) * a.N * (int64_t)D;
      qblk = a.q16 + (bh * a.N + 64 * (int64_t)i) * D;
      const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (nband <= kBand) {
        mode = 1;
        // the band's blocks, ascending, one per lane; their exact keys; each
        // lane counts the band blocks ranked before its own
        int base = 0;
#pragma unroll
        for (int t = 0; t < KPL; t++) {
          const bool in = key[t] >= Tlo && key[t] <= Thi;
          const uint64_t bal = __ballot(in);
          if (in) band_blk[base + __popcll(bal & lower)] = lane + 64 * t;
          base += __popcll(bal);
        }
        // LDS is in order for one wave; the barrier keeps the compiler from
        // reordering the reads above the writes
        __builtin_amdgcn_wave_barrier();
        int myj = 0;
        uint64_t myk = 0;
        if (lane < nband) {
          myj = band_blk[lane];
          myk = order_key64(exact_score_kind<D>(a.kind, qrow, kT, nb, qblk, kh, myj));
          band_key[lane] = myk;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < nband) {
          int rank = 0;
          for (int m = 0; m < nband; m++) {
            const uint64_t km = band_key[m];
            rank += (km > myk || (km == myk && band_blk[m] < myj)) ? 1 : 0;
          }
          decided[myj] = rank < take ? 1 : 0;
        }
        __builtin_amdgcn_wave_barrier();
      } else {
        mode = 2;
        // a wide band: the take-th largest exact key T64 by a bitwise search
        // below the bits its keys share (exact scores recomputed per pass)
        uint64_t mx = 0, mn = ~0ull;
#pragma unroll
        for (int t = 0; t < KPL; t++) {
          if (key[t] >= Tlo && key[t] <= Thi) {
            const uint64_t k64 = order_key64(exact_score_kind<D>(a.kind, qrow, kT, nb, qblk, kh, lane + 64 * t));
            mx = k64 > mx ? k64 : mx;
            mn = k64 < mn ? k64 : mn;
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const uint64_t ox = __shfl_xor(mx, off, 64), on = __shfl_xor(mn, off, 64);
          mx = ox > mx ? ox : mx;
          mn = on < mn ? on : mn;
        }
        const uint64_t diff = mx ^ mn;
        uint64_t t64 = mx;
        if (diff) {
          const int top = 63 - __builtin_clzll(diff);
          t64 = mx & ~((top == 63) ? ~0ull : ((2ull << top) - 1ull));
          for (int bit = top; bit >= 0; bit--) {
            const uint64_t c = t64 | (1ull << bit);
            int n = 0;
#pragma unroll
            for (int t = 0; t < KPL; t++) {
              const bool in = key[t] >= Tlo && key[t] <= Thi;
              uint64_t k64 = 0;
              if (in) k64 = order_key64(exact_score_kind<D>(a.kind, qrow, kT, nb, qblk, kh, lane + 64 * t));
              n += __popcll(__ballot(in && k64 >= c));
            }
            if (n >= take) t64 = c;
          }
        }
        int gt64 = 0;
#pragma unroll
        for (int t = 0; t < KPL; t++) {
          const bool in = key[t] >= Tlo && key[t] <= Thi;
          uint64_t k64 = 0;
          if (in) k64 = order_key64(exact_score_kind<D>(a.kind, qrow, kT, nb, qblk, kh, lane + 64 * t));
          gt64 += __popcll(__ballot(in && k64 > t64));
        }
        T64 = t64;
        take_eq64 = take - gt64;  // lowest-index blocks with key == T64
      }
    }
  }

  // emit: FP16 list (kk entries) ascending, then the FP4 list ascending.
  // Blocks go in ascending order j = lane + 64 t, so a block's position is
  // the count of earlier same-list blocks: whole earlier steps (scalar
  // running counts) plus the lower lanes of this step (mbcnt).
  int before16 = 0, eq_seen = 0;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int t = 0; t < KPL; t++) {
    if (64 * t >= nv) break;  // wave-uniform
    const int j = lane + 64 * t;
    const bool valid = j < nv, forced = (j == 0 || j == i);
    bool sel;
    if (!scored) {
      sel = forced || kextra > 0;  // kextra > 0 here means every valid block
    } else {
      // a nonzero key is a valid, non-forced block; Tlo is nonzero
      const bool band = key[t] >= Tlo && key[t] <= Thi;
      sel = forced || key[t] > Thi;
      if (mode == 0) {
        sel = sel || band;  // the whole band is taken
      } else if (mode == 1) {
        if (band) sel = decided[j] != 0;
      } else {
        // (mode is wave-uniform: the ballot below runs on the whole wave)
        uint64_t k64 = 0;
        if (band) k64 = order_key64(exact_score_kind<D>(a.kind, qrow, kT, nb, qblk, kh, j));
        sel = sel || k64 > T64;
        const bool tie64 = band && k64 == T64;
        const uint64_t tb = __ballot(tie64);
        if (tie64) sel = eq_seen + __popcll(tb & lower) < take_eq64;
        eq_seen += __popcll(tb);
      }
    }
    const uint64_t sb = __ballot(valid && sel);
    const int p16 = before16 + __popcll(sb & lower);
    // finite scores select exactly kk blocks, so every position is below
    // nv; non-finite inputs (outside the contract) may select fewer, and
    // their positions past the row are dropped rather than written
    const int pos = sel ? p16 : (int)kk + (j - p16);
    if (valid && pos < nv) out[pos] = j;
    before16 += __popcll(sb);
  }
  if (lane == 0) a.n16[row] = (int)kk;
}

// Query blocks [i_lo, i_lo + i_span) of every (b, h), with KPL keys per lane
// (KPL >= ceil(valid blocks / 64) for every row of the range).
template <int D, int KPL>
static hipError_t launch_select_kpl(const SelectArgs &a, hipStream_t st, const int i_lo, const int i_span) {
  const int nb = a.N / 64;
  constexpr int waves = kSelThreads / 64;
  const size_t lds = waves * select_lds_per_wave(nb);
  const void *fn = (const void *)select_kernel<D, KPL>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.Hq * i_span;
  const unsigned grid = (unsigned)((rows + waves - 1) / waves);
  hipLaunchKernelGGL((select_kernel<D, KPL>), dim3(grid), dim3(kSelThreads), lds, st, a, i_lo, i_span);
  return hipGetLastError();
}

// The rows whose valid blocks need at most KPL keys per lane: causal rows
// [64 KPL / 2, 64 KPL) (all rows from 0 for KPL = 1) or, non-causal, every row.
template <int D, int KPL>
static hipError_t launch_select_class(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  if (!a.causal) return launch_select_kpl<D, KPL>(a, st, 0, nb);
  const int lo = KPL == 1 ? 0 : 64 * (KPL / 2), hi = min(nb, 64 * KPL);
  if (lo >= hi) return hipSuccess;
  return launch_select_kpl<D, KPL>(a, st, lo, hi - lo);
}

// The block scores of a.kind into a.idx (fp32 bits at the list positions);
// the means they need go to a.qbar / a.kbarT first.
template <int D>
static hipError_t launch_scores_d(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  auto grid = [](int64_t work) {
    int64_t b = (work + 255) / 256;
    return (unsigned)(b > 256 * 64 ? 256 * 64 : b);
  };
  const int64_t BHq = (int64_t)a.B * a.Hq, BHk = (int64_t)a.B * a.Hkv;
  hipError_t e;
  if (a.kind == kScoreNormWeighted) {
    hipLaunchKernelGGL(normw_pool_kernel<false>, dim3((unsigned)(BHq * nb)), dim3(128), 0, st, a.q16, a.qbar, a.N, D);
    hipLaunchKernelGGL(normw_pool_kernel<true>, dim3((unsigned)(BHk * nb)), dim3(128), 0, st, a.k16, a.kbarT, a.N, D);
  } else if (a.kind != kScoreBlockMax) {
    hipLaunchKernelGGL(pool_kernel<false>, dim3(grid(BHq * nb * D)), dim3(256), 0, st, a.q16, a.qbar, BHq, a.N, D);
    if (a.kind == kScorePooled)
      hipLaunchKernelGGL(pool_kernel<true>, dim3(grid(BHk * nb * D)), dim3(256), 0, st, a.k16, a.kbarT, BHk, a.N, D);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int tn = (nb + 63) / 64;
  const int tiles = a.causal ? tn * (tn + 1) / 2 : tn * tn;
  if (a.kind == kScorePooled || a.kind == kScoreNormWeighted) {
    if ((e = hipFuncSetAttribute((const void *)score_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kScoreLds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(score_kernel<D>, dim3((unsigned)(BHq * tiles)), dim3(kScoreThreads), kScoreLds, st, a, tiles,
                       tn);
  } else {
    const int lds = D * (kQStride + 64) * 8;
    const void *fn = a.kind == kScoreMaxPooled ? (const void *)maxpool_score_kernel<D>
                                               : (const void *)blockmax_score_kernel<D>;
    if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    if (a.kind == kScoreMaxPooled) {
      hipLaunchKernelGGL(maxpool_score_kernel<D>, dim3((unsigned)(BHq * tiles)), dim3(kScoreThreads), lds, st, a,
                         tiles, tn);
    } else {
      const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
      const int64_t work = BHq * per;
      const unsigned g = (unsigned)(work < 65536 * 16 ? work : 65536 * 16);  // grid stride beyond 1M workgroups
      hipLaunchKernelGGL(blockmax_score_kernel<D>, dim3(g), dim3(kScoreThreads), lds, st, a, per);
    }
  }
  return hipGetLastError();
}

// The selection's pooled-mean scores: the means, their norms, then the
// fp32 chains (score32_kernel) into a.idx.
template <int D>
static hipError_t launch_scores32_d(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  auto grid = [](int64_t work) {
    int64_t b = (work + 255) / 256;
    return (unsigned)(b > 256 * 64 ? 256 * 64 : b);
  };
  const int64_t BHq = (int64_t)a.B * a.Hq, BHk = (int64_t)a.B * a.Hkv;
  hipLaunchKernelGGL(pool_kernel<false>, dim3(grid(BHq * nb * D)), dim3(256), 0, st, a.q16, a.qbar, BHq, a.N, D);
  hipLaunchKernelGGL(pool_kernel<true>, dim3(grid(BHk * nb * D)), dim3(256), 0, st, a.k16, a.kbarT, BHk, a.N, D);
  hipLaunchKernelGGL(qnorm_kernel<D>, dim3((unsigned)((BHq * nb + 255) / 256)), dim3(256), 0, st, a.qbar, a.qn,
                     BHq * nb);
  hipLaunchKernelGGL(knorm_kernel<D>, dim3((unsigned)((BHk * nb + 255) / 256)), dim3(256), 0, st, a.kbarT, a.kn, nb,
                     BHk * nb);
  hipLaunchKernelGGL(knmax_kernel, dim3((unsigned)BHk), dim3(256), 0, st, a.kn, a.knmax, nb);
  const int tn = (nb + kS32Tile - 1) / kS32Tile;
  const int tiles = a.causal ? tn * (tn + 1) / 2 : tn * tn;
  hipLaunchKernelGGL(score32_kernel<D>, dim3((unsigned)(BHq * tiles)), dim3(256), 0, st, a, tiles, tn);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_select_d(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  if (a.ppm > 0) {
    const hipError_t e = a.kind == kScorePooled ? launch_scores32_d<D>(a, st) : launch_scores_d<D>(a, st);
    if (e != hipSuccess) return e;
  }
  const int kpl = (nb + 63) / 64;
  if (!a.causal) {
    if (kpl <= 1) return launch_select_class<D, 1>(a, st);
    if (kpl <= 2) return launch_select_class<D, 2>(a, st);
    if (kpl <= 4) return launch_select_class<D, 4>(a, st);
    if (kpl <= 8) return launch_select_class<D, 8>(a, st);
    if (kpl <= 16) return launch_select_class<D, 16>(a, st);
    if (kpl <= 32) return launch_select_class<D, 32>(a, st);
    if (kpl <= 64) return launch_select_class<D, 64>(a, st);
    return launch_select_class<D, 128>(a, st);
  }
  // causal: row i has i + 1 valid blocks, so each power-of-two class of
  // rows gets the smallest KPL that holds them (the short rows do not pay
  // for the longest row's key slots)
  hipError_t e;
  if ((e = launch_select_class<D, 1>(a, st)) != hipSuccess) return e;
  if ((e = launch_select_class<D, 2>(a, st)) != hipSuccess) return e;
  if ((e = launch_select_class<D, 4>(a, st)) != hipSuccess) return e;
  if ((e = launch_select_class<D, 8>(a, st)) != hipSuccess) return e;
  if ((e = launch_select_class<D, 16>(a, st)) != hipSuccess) return e;
  if ((e = launch_select_class<D, 32>(a, st)) != hipSuccess) return e;
  if ((e = launch_select_class<D, 64>(a, st)) != hipSuccess) return e;
  return launch_select_class<D, 128>(a, st);
}

hipError_t launch_select(const SelectArgs &a, hipStream_t st) {
  return a.d == 64 ? launch_select_d<64>(a, st) : launch_select_d<128>(a, st);
}

hipError_t launch_block_scores(const SelectArgs &a, hipStream_t st) {
  return a.d == 64 ? launch_scores_d<64>(a, st) : launch_scores_d<128>(a, st);
}

// ---------------------------------------------------------------------------
// Selection without a caller workspace: the pooled means live in `scratch`,
// a static device array (one copy per GPU, held until the process ends).
// Host code never passes the array's name to a kernel (in host code it is a
// stand-in, not a device address): the first call on each device looks up
// the array's device address with hipGetSymbolAddress, with that device
// current, and every call uses that pointer.  The device is the stream's
// (the current device for the default stream), so a stream of another GPU
// than the current one gets that GPU's copy.  Calls on one GPU share the
// array, so calls that overlap in time on one GPU race; each call rewrites
// every pooled mean it reads, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kSelectScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t launch_select_scratch(SelectArgs a, hipStream_t st) {
  int dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *ptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      int cur = 0;
      if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;  // the caller's device again
      if (e != hipSuccess) return e;
      if (back != hipSuccess) return back;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  select_layout(a, (float *)ptr);
  return launch_select(a, st);
}

}  // namespace thrift
