// Issue costs of the instructions the FP4 attention step is made of, on
// gfx950, in shader-clock cycles (s_memtime around each loop), and how far
// the step's MFMAs and its VALU work overlap.  A standalone measurement
// program: it shares nothing with the library and its numbers are the ones
// the ALU roofline of the FP4 kernel is priced with.
//
// Part 1: SIMD cycles per wave64 instruction.  Every CU runs 3 workgroups of
// 4 waves (3 waves per SIMD, as the FP4 kernel; pinned by LDS), each wave 16
// independent chains of the instruction, so issue rate, not latency, is
// measured.  Workgroups reach a CU over tens of microseconds, so every
// kernel runs twice, at L and 2L loop trips, and the cost is the difference
// of the two kernel times (HIP events) at the measured clock over the work
// the extra L trips add per SIMD: ramp-up, launch and tail cancel.
// Part 2: MFMA cycles per instruction under the same occupancy (dependent
// chain and 4 independent accumulators).
// Part 3: one 64-key FP4 block of one wave (32 query rows): 4 scaled MFMAs for
// S, 32 x (fma, exp2), a 32-term row sum, the max tree, 16 FP4 pack
// converts, 4 scaled MFMAs into the accumulator; run as MFMA work only, as
// VALU work only, and whole (serially dependent, as in the kernel).  The
// clock of each run is the ratio of s_memtime to s_memrealtime (100 MHz).
//
// `isa_costs hbm R W` instead measures plain HBM traffic: one kernel reads R
// bytes and writes W bytes (16-byte vector accesses, grid-stride, 8 x 256
// workgroups per CU), and prints one JSON line with the rate (R + W) / time:
// the ceiling a kernel with that byte mix (e.g. the quantizer's) can reach.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

namespace {

constexpr int kWG = 768;  // 3 workgroups of 256 threads per CU
// Dynamic LDS per workgroup (unused): 3 fit in a CU's 160 KB, 4 do not, so
// every CU holds exactly 3 workgroups (3 waves per SIMD) whatever the
// kernels' register counts would allow.
constexpr int kLdsPin = 48 * 1024;
constexpr int kIt = 2048;     // L: loop trips (16 instructions each) in parts 1 and 2
constexpr int kBlocks = 1024;  // L: blocks per wave in part 3

__device__ unsigned long long g_cyc[kWG * 4], g_wall[kWG * 4];

__device__ __forceinline__ void record(const unsigned long long c0, const unsigned long long w0) {
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  if ((threadIdx.x & 63) == 0) {
    g_cyc[blockIdx.x * 4 + (threadIdx.x >> 6)] = c1 - c0;
    g_wall[blockIdx.x * 4 + (threadIdx.x >> 6)] = w1 - w0;
  }
}

enum Op { kFma, kAdd, kMax, kMax3, kExp, kPack, kIntXor, kFmaCvtU32, kMfmaChain, kMfma4, kMfmaF16, kMax3U32 };

template <int OP>
__global__ __launch_bounds__(256) void op_kernel(float *o, float s, const int trips) {
  float a[16], b[16];
  uint32_t u[16];
  float16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const int8v A = {(int)threadIdx.x, 1, 2, 3, 0, 0, 0, 0}, B = {5, 6, 7, (int)threadIdx.x, 0, 0, 0, 0};
  for (int i = 0; i < 16; i++) a[i] = s + threadIdx.x * 1e-3f + i, b[i] = a[i] * 0.5f, u[i] = threadIdx.x + i;
  __syncthreads();
  const unsigned long long t0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < trips; it++) {
    if (OP == kMfmaChain || OP == kMfma4) {
      // 16 MFMAs per trip: one accumulator, or four in turn
#pragma unroll
      for (int m = 0; m < 4; m++) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c0, 4, 4, 0, 127, 0, 127);
        if (OP == kMfmaChain) {
          c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B, A, c0, 4, 4, 0, 127, 0, 127);
          c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, A, c0, 4, 4, 0, 127, 0, 127);
          c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B, B, c0, 4, 4, 0, 127, 0, 127);
        } else {
          c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B, A, c1, 4, 4, 0, 127, 0, 127);
          c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, A, c2, 4, 4, 0, 127, 0, 127);
          c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(B, B, c3, 4, 4, 0, 127, 0, 127);
        }
      }
      continue;
    }
    if (OP == kMfmaF16) {
      typedef _Float16 h8 __attribute__((ext_vector_type(8)));
      const h8 ha = __builtin_bit_cast(h8, int4v{A[0], A[1], A[2], A[3]});
      const h8 hb = __builtin_bit_cast(h8, int4v{B[0], B[1], B[2], B[3]});
#pragma unroll
      for (int m = 0; m < 4; m++) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, hb, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb, ha, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb, hb, c3, 0, 0, 0);
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (OP == kFma) a[i] = fmaf(a[i], 0.9999f, b[i]);
      if (OP == kAdd) a[i] = a[i] + b[i];
      if (OP == kMax) asm volatile("v_max_f32 %0, %1, %2" : "=v"(a[i]) : "v"(a[i]), "v"(b[i]));  // kept as written
      if (OP == kMax3) a[i] = fmaxf(fmaxf(-a[i], b[i]), b[(i + 1) & 15]);
      if (OP == kExp) a[i] = __builtin_amdgcn_exp2f(a[i]);
      if (OP == kPack) u[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u[i], a[i], b[i], 0.5f, 1);
      if (OP == kIntXor) u[i] ^= u[(i + 5) & 15];
      if (OP == kFmaCvtU32) b[i] = (float)(uint32_t)fmaf(b[i], 1.0001f, 3.0f);
      if (OP == kMax3U32) u[i] = max(max(u[i] ^ 0x5a5a5a5au, (uint32_t)i), u[(i + 1) & 15]);
    }
  }
  record(t0, w0);
  float r = 0;
  for (int i = 0; i < 16; i++) r += a[i] + b[i] + (float)u[i] + c0[i] + c1[i] + c2[i] + c3[i];
  o[blockIdx.x * 256 + threadIdx.x] = r;
}

// ---- part 3: the FP4 block
__device__ __forceinline__ void block_qk(const int4v base, const int4v (&q)[2], float16v (&s)[2]) {
#pragma unroll
  for (int blk = 0; blk < 2; blk++) {
#pragma unroll
    for (int r = 0; r < 16; r++) s[blk][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      const int4v kv = base ^ (blk * 2 + kk);
      const int8v a8 = {kv[0], kv[1], kv[2], kv[3], 0, 0, 0, 0};
      const int8v b8 = {q[kk][0], q[kk][1], q[kk][2], q[kk][3], 0, 0, 0, 0};
      s[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, s[blk], 4, 4, 0, 120, 0, 120);
    }
  }
}

__device__ __forceinline__ void block_softmax(float16v (&s)[2], const float M, const float c, float &l,
                                              uint32_t (&pw)[4]) {
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s[0][r] = __builtin_amdgcn_exp2f(fmaf(s[0][r], c, -M));
    s[1][r] = __builtin_amdgcn_exp2f(fmaf(s[1][r], c, -M));
    l0 += s[0][r];
    l1 += s[1][r];
  }
  l += l0 + l1;
  float m[4] = {fmaxf(s[0][0], s[0][1]), fmaxf(s[0][8], s[0][9]), fmaxf(s[1][0], s[1][1]), fmaxf(s[1][8], s[1][9])};
#pragma unroll
  for (int r = 2; r < 8; r += 2) {
    m[0] = fmaxf(fmaxf(m[0], s[0][r]), s[0][r + 1]);
    m[1] = fmaxf(fmaxf(m[1], s[0][8 + r]), s[0][9 + r]);
    m[2] = fmaxf(fmaxf(m[2], s[1][r]), s[1][r + 1]);
    m[3] = fmaxf(fmaxf(m[3], s[1][8 + r]), s[1][9 + r]);
  }
  const float div = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])) * 0.25f;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    const int blk = w >> 1, r0 = 8 * (w & 1);
    uint32_t x = __float_as_uint(s[blk][r0]);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[blk][r0 + 0], s[blk][r0 + 1], div, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[blk][r0 + 2], s[blk][r0 + 3], div, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[blk][r0 + 4], s[blk][r0 + 5], div, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, s[blk][r0 + 6], s[blk][r0 + 7], div, 3);
    pw[w] = x;
  }
}

__device__ __forceinline__ void block_pv(const uint32_t (&pw)[4], const int4v base, float16v (&acc)[4]) {
  const int8v pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], 0, 0, 0, 0};
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    const int4v vv = base + cb;
    const int8v a8 = {vv[0], vv[1], vv[2], vv[3], 0, 0, 0, 0};
    acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, pb, acc[cb], 4, 4, 0, 120, 0, 120);
  }
}

enum Mode { kBlockMfma, kBlockValu, kBlockWhole };

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void block_kernel(
    float *o, const int4v *src, const float c, const float M, const int blocks) {
  const int lane = threadIdx.x & 63;
  const int4v q[2] = {src[lane], src[64 + lane]};
  float16v acc[4] = {};
  float l = 0.f;
  __syncthreads();
  const unsigned long long t0 = clock64(), w0 = wall_clock64();
  if (MODE == kBlockValu) {
    float16v s[2];
#pragma unroll
    for (int r = 0; r < 16; r++) s[0][r] = 0.01f * r - lane, s[1][r] = 0.02f * r + lane;
    uint32_t x = 0;
    for (int j = 0; j < blocks; j++) {
      uint32_t pw[4];
      block_softmax(s, M, c, l, pw);
      x ^= pw[0] ^ pw[1] ^ pw[2] ^ pw[3];
    }
    acc[0][0] = (float)x;
  } else {
    for (int j = 0; j < blocks; j++) {
      const int4v base = src[128 + ((j * 7 + lane) & 255)];
      float16v s[2];
      block_qk(base, q, s);
      uint32_t pw[4];
      if (MODE == kBlockWhole) {
        block_softmax(s, M, c, l, pw);
      } else {
        pw[0] = __float_as_uint(s[0][0]), pw[1] = __float_as_uint(s[0][8]);
        pw[2] = __float_as_uint(s[1][0]), pw[3] = __float_as_uint(s[1][8]);
      }
      block_pv(pw, base, acc);
    }
  }
  record(t0, w0);
  float r = l;
#pragma unroll
  for (int cb = 0; cb < 4; cb++)
#pragma unroll
    for (int i = 0; i < 16; i++) r += acc[cb][i];
  o[blockIdx.x * 256 + threadIdx.x] = r;
}

struct Timed {
  double ms, ghz;  // kernel time (HIP events), clock over the run (s_memtime / s_memrealtime)
};

// One warm launch, then one timed launch of `launch(n)`.
template <typename F>
Timed timed(F launch, const int n) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return {-1.0, 0.0};
  launch(n);
  (void)hipEventRecord(e0, 0);
  launch(n);
  (void)hipEventRecord(e1, 0);
  if (hipDeviceSynchronize() != hipSuccess) return {-1.0, 0.0};
  float ms = 0.0f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  static unsigned long long hc[kWG * 4], hw[kWG * 4];
  if (hipMemcpyFromSymbol(hc, HIP_SYMBOL(g_cyc), sizeof hc) != hipSuccess ||
      hipMemcpyFromSymbol(hw, HIP_SYMBOL(g_wall), sizeof hw) != hipSuccess)
    return {-1.0, 0.0};
  double sc = 0, sw = 0;
  for (int i = 0; i < kWG * 4; i++) sc += (double)hc[i], sw += (double)hw[i];
  int wall_khz = 100000;
  (void)hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0);
  return {(double)ms, sc / sw * wall_khz * 1e-6};
}

// SIMD cycles per unit of work: the extra time of 2L over L trips at the
// clock of the 2L run, over the extra units per SIMD (3 waves x L x units
// per trip).
template <typename F>
bool differential(F launch, const int L, const double units_per_trip, double &cycles, double &ghz) {
  const Timed a = timed(launch, L), b = timed(launch, 2 * L);
  if (a.ms < 0 || b.ms < 0) return false;
  ghz = b.ghz;
  cycles = (b.ms - a.ms) * 1e6 * b.ghz / (3.0 * L * units_per_trip);
  return true;
}


// ---- HBM: read nr and write nw 16-byte chunks (grid-stride); a written
// chunk takes the loaded chunk of the same index when there is one
__global__ __launch_bounds__(256) void hbm_kernel(const int4v *__restrict__ a, int4v *__restrict__ b, const size_t nr,
                                                  const size_t nw) {
  const size_t n = nr > nw ? nr : nw, stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    int4v v = {(int)i, 1, 2, 3};
    if (i < nr) v = a[i];
    if (i < nw) b[i] = v;
    else if (v[0] == 0x7fffffff && v[1] == -1) b[0] = v;  // keeps the read live; never true for the fill below
  }
}

int hbm_main(const size_t rbytes, const size_t wbytes) {
  const size_t nr = rbytes / 16, nw = wbytes / 16;
  int4v *a = nullptr, *b = nullptr;
  if (hipMalloc(&a, (nr ? nr : 1) * 16) != hipSuccess || hipMalloc(&b, (nw ? nw : 1) * 16) != hipSuccess) {
    std::printf("{\"error\": \"device allocation failed\"}\n");
    return 1;
  }
  if (hipMemset(a, 0x11, (nr ? nr : 1) * 16) != hipSuccess) return 1;
  int ncu = 256;
  (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0);
  const dim3 grid(8 * ncu);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  const int reps = 10;
  hipLaunchKernelGGL(hbm_kernel, grid, dim3(256), 0, 0, a, b, nr, nw);
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; r++) hipLaunchKernelGGL(hbm_kernel, grid, dim3(256), 0, 0, a, b, nr, nw);
  (void)hipEventRecord(e1, 0);
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  float ms = 0.0f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  ms /= reps;
  std::printf("{\"read_bytes\": %zu, \"write_bytes\": %zu, \"ms\": %.4f, \"GBps\": %.1f}\n", nr * 16, nw * 16,
              ms, (double)(nr + nw) * 16 / (ms * 1e-3) / 1e9);
  hipFree(a);
  hipFree(b);
  return 0;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc == 4 && !std::strcmp(argv[1], "hbm")) return hbm_main(std::strtoull(argv[2], nullptr, 10), std::strtoull(argv[3], nullptr, 10));
  float *o = nullptr;
  int4v *src = nullptr;
  if (hipMalloc(&o, kWG * 256 * sizeof(float)) != hipSuccess || hipMalloc(&src, 384 * sizeof(int4v)) != hipSuccess) {
    std::printf("device allocation failed\n");
    return 1;
  }
  int h[384 * 4];
  for (int i = 0; i < 384 * 4; i++) h[i] = (int)((unsigned)i * 2654435761u) & 0x77777777;
  if (hipMemcpy(src, h, sizeof h, hipMemcpyHostToDevice) != hipSuccess) return 1;

  std::printf("gfx950 issue costs, 3 waves per SIMD (768 workgroups of 256 threads, 3 per CU), shader-clock cycles\n");
  std::printf("(difference of kernel times at L and 2L loop trips, at the clock measured over the 2L run)\n");
  struct {
    void (*k)(float *, float, int);
    const char *name;
  } ops[] = {
      {op_kernel<kFma>, "v_fma_f32"},
      {op_kernel<kAdd>, "v_add_f32"},
      {op_kernel<kMax>, "v_max_f32"},
      {op_kernel<kMax3>, "v_max3_f32"},
      {op_kernel<kExp>, "v_exp_f32"},
      {op_kernel<kPack>, "v_cvt_scalef32_pk_fp4_f32"},
      {op_kernel<kIntXor>, "v_xor_b32 (an integer VALU op)"},
      {op_kernel<kFmaCvtU32>, "v_fma_f32 + v_cvt_u32_f32 + v_cvt_f32_u32 (one each)"},
      {op_kernel<kMfmaChain>, "v_mfma_scale_f32_32x32x64_f8f6f4 (fp4), one chain"},
      {op_kernel<kMfma4>, "v_mfma_scale_f32_32x32x64_f8f6f4 (fp4), 4 chains"},
      {op_kernel<kMfmaF16>, "v_mfma_f32_32x32x16_f16, 4 chains"},
      {op_kernel<kMax3U32>, "v_xor_b32 + v_max3_u32 (one each)"},
  };
  for (const auto &op : ops) {
    double cyc, ghz;
    if (!differential([&](int n) { hipLaunchKernelGGL(op.k, dim3(kWG), dim3(256), kLdsPin, 0, o, 1.0f, n); }, kIt,
                      16.0, cyc, ghz))
      return 2;
    std::printf("  %-56s %7.2f SIMD cycles per instruction  (clock %.3f GHz)\n", op.name, cyc, ghz);
  }
  std::printf("FP4 block of one wave (32 query rows x 64 keys), SIMD cycles per block-wave\n");
  struct {
    void (*k)(float *, const int4v *, float, float, int);
    const char *name;
  } blocks[] = {{block_kernel<kBlockMfma>, "8 scaled FP4 MFMAs only"},
                {block_kernel<kBlockValu>, "softmax VALU only (exp2, sum, max, FP4 pack)"},
                {block_kernel<kBlockWhole>, "whole block (QK -> softmax -> PV)"}};
  for (const auto &b : blocks) {
    double cyc, ghz;
    if (!differential(
            [&](int n) { hipLaunchKernelGGL(b.k, dim3(kWG), dim3(256), kLdsPin, 0, o, src, 0.01f, 3.0f, n); },
            kBlocks, 1.0, cyc, ghz))
      return 2;
    std::printf("  %-56s %7.1f cycles  (clock %.3f GHz)\n", b.name, cyc, ghz);
  }
  std::printf("status %s\n", hipGetErrorString(hipDeviceSynchronize()));
  hipFree(o);
  hipFree(src);
  return 0;
}
