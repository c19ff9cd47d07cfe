// Step 2 of the ThriftAttention path ("ThriftAttention: Selective Mixed
// Precision for Long-Context FP4 Attention", abstract: a heuristic rapidly
// selects a small number of important query-key block pairs for FP16).
//
// Heuristic: mean-pool every 64-row block of Q (per query head) and K (per
// KV head); score the pair (i, j) by the fp64 dot product of the means taken
// in channel order; per (b, h_q, i) keep the first and diagonal key blocks
// and the best-scoring others up to ceil(frac * valid blocks) in total.
//
// Bit-exactness: the pooled sums of 64 fp16 values are exact in fp64 (they
// need at most 46 significant bits), so their order does not matter; each
// product of two fp32 means is exact in fp64, so a sequential fma chain in
// channel order gives the same bits as any sequential multiply-add in that
// order.
#include "thrift_internal.h"

namespace thrift {

// One thread per (head row-block, channel).  Q means are written row-major
// [BH, nb, d]; K means transposed [BH, d, nb] so that the scoring kernel
// reads them coalesced.
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

// Order-preserving map of a double to uint64 (larger value -> larger key);
// -0 is folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint64_t order_key(double s) {
  if (s == 0.0) s = 0.0;
  uint64_t u = __double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kSelThreads = 256;

// Inclusive prefix sum of one value per lane over the wave (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

// Inclusive prefix sum of one value per thread over the block (kSelThreads
// threads, in thread order); also returns the total.  `wsum` holds one int
// per wave.  Contains two barriers.
__device__ int block_inclusive_scan(int v, int *wsum, int &total) {
  const int w = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if ((threadIdx.x & 63) == 63) wsum[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int u = 0; u < kSelThreads / 64; u++) {
    before += (u < w) ? wsum[u] : 0;
    all += wsum[u];
  }
  total = all;
  __syncthreads();  // wsum may be rewritten by the next call
  return before + x;
}

// Score of query block i against key block j: the fp64 fma chain over the
// D channels in order.  The K means are loaded 16 channels at a time, so 16
// loads are in flight before their fmas.
template <int D>
__device__ __forceinline__ double block_score(const double *qrow, const float *kT, const int nb, const int j) {
  double s = 0.0;
#pragma unroll 1
  for (int c0 = 0; c0 < D; c0 += 16) {
    float kv[16];
#pragma unroll
    for (int u = 0; u < 16; u++) kv[u] = kT[(int64_t)(c0 + u) * nb + j];
#pragma unroll
    for (int u = 0; u < 16; u++) s = fma(qrow[c0 + u], (double)kv[u], s);
  }
  return s;
}

// One workgroup per (b, h_q, query block i).
template <int D>
__global__ __launch_bounds__(kSelThreads) void score_select_kernel(SelectArgs a) {
  extern __shared__ uint64_t keys[];  // [n_valid]
  __shared__ double qrow[128];
  __shared__ int hist[256];
  __shared__ int wsum[kSelThreads / 64];
  __shared__ int s_digit, s_above, s_count;

  const int nb = a.N / 64;
  const int64_t row = blockIdx.x;  // = (b*Hq + h)*nb + i
  const int i = (int)(row % nb);
  const int64_t bh = row / nb;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = (int)((int64_t)h * a.Hkv / a.Hq);
  const int nv = a.causal ? i + 1 : nb;
  const int tid = threadIdx.x;
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  int32_t *out = a.idx + bh * per + (a.causal ? (int64_t)i * (i + 1) / 2 : (int64_t)i * nb);

  if (a.ppm == 0) {  // no FP16 blocks: the FP4 list is every valid block
    for (int j = tid; j < nv; j += kSelThreads) out[j] = j;
    if (tid == 0) a.n16[row] = 0;
    return;
  }
  const int nforced = (i == 0) ? 1 : 2;
  int64_t want = (a.ppm * nv + 999999) / 1000000;
  int64_t kk = want > nforced ? want : nforced;
  if (kk > nv) kk = nv;
  const int kextra = (int)kk - nforced;  // best non-forced blocks to add

  // contiguous chunk of block indices per thread (keeps index order for scans)
  const int chunk = (nv + kSelThreads - 1) / kSelThreads;
  const int j0 = tid * chunk, j1 = min(nv, j0 + chunk);

  if (kextra > 0 && kextra < nv - nforced) {
    for (int c = tid; c < a.d; c += kSelThreads) qrow[c] = (double)a.qbar[row * a.d + c];
    __syncthreads();
    // scores: strided j for coalesced reads of the transposed K means
    const float *kT = a.kbarT + (int64_t)(b * a.Hkv + g) * a.d * nb;
    for (int j = tid; j < nv; j += kSelThreads) keys[j] = order_key(block_score<D>(qrow, kT, nb, j));
    __syncthreads();
    // radix select (8 bits per pass, most significant first) of the kextra-th
    // largest key among the non-forced blocks.  After a pass, the candidates
    // whose key starts with `prefix` (under pmask) hold the `remaining`
    // largest not yet taken; if they are exactly that many, every one of
    // them is taken and the search stops early.
    uint64_t prefix = 0, pmask = 0;
    int remaining = kextra;
    for (int pass = 0; pass < 8; pass++) {
      const int shift = 56 - 8 * pass;
      hist[tid] = 0;  // kSelThreads == 256 bins
      __syncthreads();
      for (int j = tid; j < nv; j += kSelThreads) {
        if (j == 0 || j == i) continue;
        const uint64_t kj = keys[j];
        if ((kj & pmask) == prefix) atomicAdd(&hist[(kj >> shift) & 255], 1);
      }
      __syncthreads();
      // the digit whose bin holds the remaining-th largest candidate: thread
      // t takes digit 255 - t, so the inclusive scan counts the candidates
      // at or above that digit; exactly one thread (a non-empty bin) crosses
      const int cnt = hist[255 - tid];
      int ncand;
      const int at_or_above = block_inclusive_scan(cnt, wsum, ncand);
      if (at_or_above >= remaining && at_or_above - cnt < remaining) {
        s_digit = 255 - tid;
        s_above = at_or_above - cnt;
        s_count = cnt;
      }
      __syncthreads();
      remaining -= s_above;
      prefix |= (uint64_t)s_digit << shift;
      pmask |= (uint64_t)255 << shift;
      const bool done = s_count == remaining;
      __syncthreads();
      if (done) break;
    }
    // prefix (under pmask) is the threshold T: take every key whose masked
    // value is > T and the `remaining` lowest-index keys whose masked value
    // is == T (all of them when the search stopped early)
    int neq = 0;
    for (int j = j0; j < j1; j++)
      if (j != 0 && j != i && (keys[j] & pmask) == prefix) neq++;
    int tot;
    int rank = block_inclusive_scan(neq, wsum, tot) - neq;
    // mark the FP16 set in the key array: 1 = FP16, 0 = FP4
    for (int j = j0; j < j1; j++) {
      uint64_t kj = keys[j];
      int sel;
      if (j == 0 || j == i)
        sel = 1;
      else if ((kj & pmask) > prefix)
        sel = 1;
      else if ((kj & pmask) == prefix)
        sel = (rank++ < remaining);
      else
        sel = 0;
      keys[j] = (uint64_t)sel;  // only this thread touches its chunk from here
    }
    __syncthreads();
  } else {
    // all non-forced blocks (kextra == nv - nforced) or none (kextra == 0)
    const uint64_t v = kextra > 0 ? 1 : 0;
    for (int j = j0; j < j1; j++) keys[j] = (j == 0 || j == i) ? 1 : v;
    __syncthreads();
  }
  // emit: FP16 list ascending, then FP4 list ascending
  int c16 = 0;
  for (int j = j0; j < j1; j++) c16 += (int)keys[j];
  int tot16;
  int p16 = block_inclusive_scan(c16, wsum, tot16) - c16;
  int p4 = tot16 + (j0 - p16);  // FP4 entries before this chunk = blocks before it minus FP16 ones
  for (int j = j0; j < j1; j++) {
    if (keys[j])
      out[p16++] = j;
    else
      out[p4++] = j;
  }
  if (tid == 0) a.n16[row] = tot16;
}

hipError_t launch_select(const SelectArgs &a, hipStream_t st) {
  const int nb = a.N / 64;
  auto grid = [](int64_t work) {
    int64_t b = (work + 255) / 256;
    return (unsigned)(b > 256 * 64 ? 256 * 64 : b);
  };
  const int64_t BHq = (int64_t)a.B * a.Hq, BHk = (int64_t)a.B * a.Hkv;
  hipLaunchKernelGGL(pool_kernel<false>, dim3(grid(BHq * nb * a.d)), dim3(256), 0, st, a.q16, a.qbar, BHq, a.N, a.d);
  hipLaunchKernelGGL(pool_kernel<true>, dim3(grid(BHk * nb * a.d)), dim3(256), 0, st, a.k16, a.kbarT, BHk, a.N, a.d);
  const size_t lds = sizeof(uint64_t) * (size_t)nb;
  const void *fn = a.d == 64 ? (const void *)score_select_kernel<64> : (const void *)score_select_kernel<128>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (a.d == 64)
    hipLaunchKernelGGL(score_select_kernel<64>, dim3((unsigned)(BHq * nb)), dim3(kSelThreads), lds, st, a);
  else
    hipLaunchKernelGGL(score_select_kernel<128>, dim3((unsigned)(BHq * nb)), dim3(kSelThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace thrift
