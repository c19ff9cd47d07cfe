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

// KPL: keys per lane, at least ceil(nb / 64).  Lane l holds blocks l + 64 t.
// LDS: nb 64-bit keys per wave for the blocks tied at the fp32 cut-off.
template <int D, int KPL>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a, int waves_per_wg) {
  extern __shared__ uint64_t tie64[];
  const int nb = a.N / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * waves_per_wg + wave;  // = (b*Hq + h)*nb + i
  if (wave >= waves_per_wg || row >= (int64_t)a.B * a.Hq * nb) return;
  const int i = (int)(row % nb);
  const int64_t bh = row / nb;
  const int nv = a.causal ? i + 1 : nb;
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  int32_t *out = a.idx + bh * per + row_offset(i, nb, a.causal);

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

  // key: order key of the block's fp32 score (0: not a candidate); blocks
  // above the cut-off T are taken, those tied with it are decided below
  uint32_t key[KPL];
  uint32_t T = 0;
  int take_eq = 0;       // how many blocks tied at T join the FP16 list
  bool exact = false;    // the tied blocks need their fp64 scores
  uint64_t T64 = 0;
  int take_eq64 = 0;
  uint64_t *tk = tie64 + (size_t)wave * nb;
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
    T = kth_largest<KPL>(key, kextra);
    int gt = 0, eq = 0;
#pragma unroll
    for (int t = 0; t < KPL; t++) {
      gt += __popcll(__ballot(key[t] > T));
      eq += __popcll(__ballot(key[t] == T));
    }
    take_eq = kextra - gt;  // 1 .. eq
    exact = take_eq < eq;
    if (exact) {
      // the fp64 scores of the tied blocks decide; among equal fp64 scores
      // the lower block index wins
      const int g = (int)((int64_t)(bh % a.Hq) * a.Hkv / a.Hq), b = (int)(bh / a.Hq);
      const float *qrow = a.qbar + row * (int64_t)D;
      const float *kT = a.kbarT + ((int64_t)b * a.Hkv + g) * D * (int64_t)nb;
      uint64_t mx = 0, mn = ~0ull;
#pragma unroll
      for (int t = 0; t < KPL; t++) {
        const int j = lane + 64 * t;
        uint64_t k64 = 0;
        if (key[t] == T) k64 = order_key64(exact_score<D>(qrow, kT, nb, j));
        if (j < nb) tk[j] = k64;
        mx = k64 > mx ? k64 : mx;
        mn = (k64 && k64 < mn) ? k64 : mn;
      }
      // this wave reads back what its other lanes wrote (LDS is in order
      // for one wave; the barrier keeps the compiler from reordering)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t ox = __shfl_xor(mx, off, 64), on = __shfl_xor(mn, off, 64);
        mx = ox > mx ? ox : mx;
        mn = on < mn ? on : mn;
      }
      // take_eq-th largest 64-bit key among the tied blocks (bitwise search
      // below the bits common to all of them)
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
            const int j = lane + 64 * t;
            n += __popcll(__ballot(j < nb && tk[j] >= c));
          }
          if (n >= take_eq) t64 = c;
        }
      }
      int gt64 = 0;
#pragma unroll
      for (int t = 0; t < KPL; t++) {
        const int j = lane + 64 * t;
        gt64 += __popcll(__ballot(j < nb && tk[j] > t64));
      }
      T64 = t64;
      take_eq64 = take_eq - gt64;  // lowest-index blocks with key == T64
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
      // a nonzero key is a valid, non-forced block; T is nonzero
      const bool tied = key[t] == T;
      sel = forced || key[t] > T;
      if (!exact) {
        sel = sel || tied;  // every tied block is taken
      } else {
        // (exact is wave-uniform: the ballot below runs on the whole wave)
        const uint64_t k64 = tied ? tk[j] : 0ull;
        sel = sel || k64 > T64;
        const bool tie64 = tied && k64 == T64;
        const uint64_t tb = __ballot(tie64);
        if (tie64) sel = eq_seen + __popcll(tb & lower) < take_eq64;
        eq_seen += __popcll(tb);
      }
    }
    const uint64_t sb = __ballot(valid && sel);
    const int p16 = before16 + __popcll(sb & lower);
    if (valid) out[sel ? p16 : (int)kk + (j - p16)] = j;
    before16 += __popcll(sb);
  }
  if (lane == 0) a.n16[row] = (int)kk;
}

template <int D, int KPL>
static hipError_t launch_select_kpl(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  int wpw = (int)(65536 / ((size_t)nb * 8));
  wpw = wpw < 1 ? 1 : (wpw > kSelThreads / 64 ? kSelThreads / 64 : wpw);
  const size_t lds = (size_t)wpw * nb * 8;
  const void *fn = (const void *)select_kernel<D, KPL>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.Hq * nb;
  const unsigned grid = (unsigned)((rows + wpw - 1) / wpw);
  hipLaunchKernelGGL((select_kernel<D, KPL>), dim3(grid), dim3(64 * wpw), lds, st, a, wpw);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_select_d(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  if (a.ppm > 0) {
    const int tn = (nb + 63) / 64;
    const int tiles = a.causal ? tn * (tn + 1) / 2 : tn * tn;
    const size_t lds = kScoreLds;
    hipError_t e = hipFuncSetAttribute((const void *)score_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    const int64_t grid = (int64_t)a.B * a.Hq * tiles;
    hipLaunchKernelGGL(score_kernel<D>, dim3((unsigned)grid), dim3(kScoreThreads), lds, st, a, tiles, tn);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int kpl = (nb + 63) / 64;
  if (kpl <= 1) return launch_select_kpl<D, 1>(a, st);
  if (kpl <= 2) return launch_select_kpl<D, 2>(a, st);
  if (kpl <= 4) return launch_select_kpl<D, 4>(a, st);
  if (kpl <= 8) return launch_select_kpl<D, 8>(a, st);
  if (kpl <= 16) return launch_select_kpl<D, 16>(a, st);
  if (kpl <= 32) return launch_select_kpl<D, 32>(a, st);
  if (kpl <= 64) return launch_select_kpl<D, 64>(a, st);
  return launch_select_kpl<D, 128>(a, st);
}

hipError_t launch_select(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  auto grid = [](int64_t work) {
    int64_t b = (work + 255) / 256;
    return (unsigned)(b > 256 * 64 ? 256 * 64 : b);
  };
  const int64_t BHq = (int64_t)a.B * a.Hq, BHk = (int64_t)a.B * a.Hkv;
  if (a.ppm > 0) {
    hipLaunchKernelGGL(pool_kernel<false>, dim3(grid(BHq * nb * a.d)), dim3(256), 0, st, a.q16, a.qbar, BHq, a.N,
                       a.d);
    hipLaunchKernelGGL(pool_kernel<true>, dim3(grid(BHk * nb * a.d)), dim3(256), 0, st, a.k16, a.kbarT, BHk, a.N,
                       a.d);
  }
  return a.d == 64 ? launch_select_d<64>(a, st) : launch_select_d<128>(a, st);
}

// ---------------------------------------------------------------------------
// Selection without a caller workspace: the pooled means live in `scratch`,
// a static device array (one copy per GPU, held until the process ends).
// Host code never passes the array's name to a kernel (in host code it is a
// stand-in, not a device address): the first call on each device looks up
// the array's device address with hipGetSymbolAddress, with that device
// current, and every call uses that pointer.  Calls on one GPU share the
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
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *ptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  a.qbar = (float *)ptr;
  a.kbarT = (float *)ptr + (size_t)a.B * a.Hq * (a.N / 64) * a.d;
  return launch_select(a, st);
}

}  // namespace thrift
