// Step 1 of the ThriftAttention path ("ThriftAttention: Selective Mixed
// Precision for Long-Context FP4 Attention", abstract: block-scaled 4-bit
// attention operands): FP16 copies of Q, K, V plus their MXFP4 codes.
// Q and K are grouped along the head dimension, V along tokens.
//
// Both kernels are HBM-bound streaming passes (2 bytes read, 2 + 1/2 + 1/32
// bytes written per element).
#include "thrift_internal.h"

namespace thrift {

// 8 input elements (fp16 or bf16 bits in a 16-byte word) -> fp32 values of
// their nearest-even fp16 roundings.
template <bool BF16>
__device__ __forceinline__ void load8_as_fp16(const int4v raw, float (&f)[8], half8 &h) {
#pragma unroll
  for (int w = 0; w < 4; w++) {
    uint32_t u = (uint32_t)raw[w];
    float lo, hi;
    if (BF16) {
      lo = __uint_as_float(u << 16);
      hi = __uint_as_float(u & 0xffff0000u);
    } else {
      lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
      hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    }
    h[2 * w] = (_Float16)lo;  // v_cvt_f16_f32: round to nearest even
    h[2 * w + 1] = (_Float16)hi;
    f[2 * w] = (float)h[2 * w];
    f[2 * w + 1] = (float)h[2 * w + 1];
  }
}

// Rows of d channels (Q or K): four lanes per 32-channel group, eight
// channels per lane.  Lanes 4m..4m+3 of a wave always belong to one group,
// and the loop bound is a multiple of 4, so the group reduction's shuffles
// only read active lanes.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_rows_kernel(const int4v *__restrict__ x, int4v *__restrict__ x16,
                                                         uint32_t *__restrict__ x4, uint8_t *__restrict__ x4s,
                                                         int64_t nlanes) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nlanes; u += stride) {
    float f[8];
    half8 h;
    load8_as_fp16<BF16>(x[u], f, h);
    x16[u] = __builtin_bit_cast(int4v, h);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(f[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int sb = mx_scale_byte(amax);
    const float div = mx_scale_divisor(sb);
    uint32_t word = 0;
    THRIFT_CVT_FP4(word, f[0], f[1], div, 0);
    THRIFT_CVT_FP4(word, f[2], f[3], div, 1);
    THRIFT_CVT_FP4(word, f[4], f[5], div, 2);
    THRIFT_CVT_FP4(word, f[6], f[7], div, 3);
    x4[u] = word;
    if ((u & 3) == 0) x4s[u >> 2] = (uint8_t)sb;
  }
}

// V: one workgroup per (b, kv head, 64-token block).  The block is staged in
// LDS channel-major; each thread then owns one (channel, 32-token group) and
// writes its FP16 run, codes and scale into the tile-major outputs.
template <bool BF16, int D>
__global__ __launch_bounds__(2 * D) void quant_v_kernel(const int4v *__restrict__ v, uint16_t *__restrict__ v16,
                                                        uint8_t *__restrict__ v4, uint8_t *__restrict__ v4s) {
  constexpr int LD = 64 + 8;  // padded row (halves) of the channel-major tile
  __shared__ _Float16 tile[D * LD];
  const int64_t blk = blockIdx.x;  // = (b*Hkv + h)*nb + n; tokens 64n.. are contiguous in v
  const int tid = threadIdx.x;
  const int4v *src = v + blk * (64 * D / 8);
  // 64*D/8 16-byte words, 2D threads -> 4 words each
#pragma unroll
  for (int it = 0; it < 4; it++) {
    const int w = tid + it * 2 * D;
    const int tok = w / (D / 8), c0 = (w % (D / 8)) * 8;
    float f[8];
    half8 h;
    load8_as_fp16<BF16>(src[w], f, h);
#pragma unroll
    for (int e = 0; e < 8; e++) tile[(c0 + e) * LD + tok] = h[e];
  }
  __syncthreads();
  const int ch = tid >> 1, grp = tid & 1;
  const _Float16 *run = tile + ch * LD + 32 * grp;
  float f[32];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; e++) {
    f[e] = (float)run[e];
    amax = fmaxf(amax, fabsf(f[e]));
  }
  // v16 tile [D][64] halves: this thread's 32 tokens are 64 contiguous bytes
  int4v *dst16 = (int4v *)(v16 + blk * (64 * D) + ch * 64 + 32 * grp);
#pragma unroll
  for (int w = 0; w < 4; w++) {
    half8 h;
#pragma unroll
    for (int e = 0; e < 8; e++) h[e] = run[8 * w + e];
    dst16[w] = __builtin_bit_cast(int4v, h);
  }
  const int sb = mx_scale_byte(amax);
  const float div = mx_scale_divisor(sb);
  uint32_t word[4] = {0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < 4; w++) {
    THRIFT_CVT_FP4(word[w], f[8 * w + 0], f[8 * w + 1], div, 0);
    THRIFT_CVT_FP4(word[w], f[8 * w + 2], f[8 * w + 3], div, 1);
    THRIFT_CVT_FP4(word[w], f[8 * w + 4], f[8 * w + 5], div, 2);
    THRIFT_CVT_FP4(word[w], f[8 * w + 6], f[8 * w + 7], div, 3);
  }
  // v4 tile [D][32 bytes]: this thread's group is 16 contiguous bytes
  int4v codes = {(int)word[0], (int)word[1], (int)word[2], (int)word[3]};
  *(int4v *)(v4 + blk * (32 * D) + ch * 32 + 16 * grp) = codes;
  v4s[blk * (2 * D) + ch * 2 + grp] = (uint8_t)sb;
}

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st) {
  const int64_t nq = (int64_t)a.B * a.Hq * a.N * a.d, nk = (int64_t)a.B * a.Hkv * a.N * a.d;
  auto rows = [&](const void *x, uint16_t *x16, uint8_t *x4, uint8_t *x4s, int64_t n) {
    const int64_t nlanes = n / 8;
    int64_t blocks = (nlanes + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 blocks per CU
    if (a.bf16)
      hipLaunchKernelGGL(quant_rows_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, (const int4v *)x,
                         (int4v *)x16, (uint32_t *)x4, x4s, nlanes);
    else
      hipLaunchKernelGGL(quant_rows_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, (const int4v *)x,
                         (int4v *)x16, (uint32_t *)x4, x4s, nlanes);
  };
  rows(a.q, a.q16, a.q4, a.q4s, nq);
  rows(a.k, a.k16, a.k4, a.k4s, nk);
  const unsigned vblocks = (unsigned)((int64_t)a.B * a.Hkv * (a.N / 64));
  if (a.d == 128) {
    if (a.bf16)
      hipLaunchKernelGGL((quant_v_kernel<true, 128>), dim3(vblocks), dim3(256), 0, st, (const int4v *)a.v, a.v16,
                         a.v4, a.v4s);
    else
      hipLaunchKernelGGL((quant_v_kernel<false, 128>), dim3(vblocks), dim3(256), 0, st, (const int4v *)a.v, a.v16,
                         a.v4, a.v4s);
  } else {
    if (a.bf16)
      hipLaunchKernelGGL((quant_v_kernel<true, 64>), dim3(vblocks), dim3(128), 0, st, (const int4v *)a.v, a.v16,
                         a.v4, a.v4s);
    else
      hipLaunchKernelGGL((quant_v_kernel<false, 64>), dim3(vblocks), dim3(128), 0, st, (const int4v *)a.v, a.v16,
                         a.v4, a.v4s);
  }
  return hipGetLastError();
}

}  // namespace thrift
