// Internal declarations shared by the HIP sources of libthrift (not part of
// the C ABI).  Device helpers for the gfx950 MXFP4 and MFMA paths.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thrift {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// Largest supported number of 64-row blocks (bounds the LDS the selection
// and attention kernels reserve per block row).
constexpr int kMaxBlocks = 8192;

// E8M0 scale byte of an MXFP4 group from the bit pattern of its largest
// magnitude (a normal or zero fp32): floor(log2 amax) - 2 + 127, clamped at
// 0 (amax = 0 or amax < 2^-124).
__device__ __forceinline__ int mx_scale_byte(float amax) {
  int biased = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  int s = biased - 2;
  return s > 0 ? s : 0;
}

// The power of two the hardware convert divides by for scale byte s (s >= 1).
// Byte 0 (2^-127, an fp32 subnormal) only occurs for groups whose values
// are all zero or below 2^-124: they take a divisor of 1 and so all-zero
// codes, where the MX rule would keep codes for values from 2^-129 up (the
// one documented departure from the rule; only re-quantized P reaches it).
__device__ __forceinline__ float mx_scale_divisor(int s) { return s > 0 ? __uint_as_float((uint32_t)s << 23) : 1.0f; }

// Two fp32 values divided by `div` and rounded to E2M1 (nearest-even,
// saturating, sign kept) into byte `sel` of `word`: low nibble = a.
// v_cvt_scalef32_pk_fp4_f32 on gfx950 computes exactly this.
#define THRIFT_CVT_FP4(word, a, b, div, sel) \
  (word) = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((word), (a), (b), (div), (sel))

struct QuantArgs {
  const void *q, *k, *v;
  uint16_t *q16, *k16, *v16;
  uint8_t *q4, *q4s, *k4, *k4s, *v4, *v4s;
  int B, Hq, Hkv, N, d;
  int bf16;
};

struct SelectArgs {
  const uint16_t *q16, *k16;
  int32_t *idx, *n16;
  float *qbar;   // [B,Hq,nb,d]
  float *kbarT;  // [B,Hkv,d,nb]
  float *qn;     // [B,Hq,nb]  Euclidean norms of the Q means, rounded up
  float *kn;     // [B,Hkv,nb] Euclidean norms of the K means, rounded up
  float *knmax;  // [B,Hkv]    largest K-mean norm over blocks 1 .. nb-1
  int B, Hq, Hkv, N, d, causal;
  int64_t ppm;
  int kind = 0;  // block score: 0 pooled mean, 1 max-pooled, 2 norm-weighted, 3 block max
};

// Selection workspace, in floats: the pooled means of Q and K, then the
// norms of both and the largest K norm of each KV head.
inline size_t select_workspace_floats(int B, int Hq, int Hkv, int N, int d) {
  const size_t nb = (size_t)(N / 64), bq = (size_t)B * Hq, bk = (size_t)B * Hkv;
  return nb * (size_t)(d + 1) * (bq + bk) + bk;
}

// Points the workspace arrays of a (shape fields set) into base.
inline void select_layout(SelectArgs &a, float *base) {
  const size_t nb = (size_t)(a.N / 64), bq = (size_t)a.B * a.Hq, bk = (size_t)a.B * a.Hkv;
  a.qbar = base;
  a.kbarT = a.qbar + bq * nb * a.d;
  a.qn = a.kbarT + bk * nb * a.d;
  a.kn = a.qn + bq * nb;
  a.knmax = a.kn + bk * nb;
}

struct AttnArgs {
  const uint16_t *q16, *k16, *v16;
  const uint8_t *q4, *q4s, *k4, *k4s, *v4, *v4s;
  const int32_t *idx, *n16;
  void *out;
  float *lse;
  float *ws;  // partial state of every row after its FP16 blocks
  int B, Hq, Hkv, N, d, causal, out_dtype;
  int rowsum;  // 0: the row sum adds the unquantized p; 1: the weights P.V uses;
               // 2: as 1, with FP4 P codes taken without an exponential
  float c;     // fl32(sm_scale * log2 e)
  // Set by the attention launcher for each FP4/redo launch: the launch
  // covers heads [hbase, hbase + hspan) of every GQA group, and its
  // workgroup w keeps its redo flag at index fbase + w.
  int hbase = 0, hspan = 0, fbase = 0;
};

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st);
hipError_t launch_select(const SelectArgs &a, hipStream_t st);
// The block scores of a.kind alone, rounded to fp32, written (as bits) into
// a.idx at the list positions (no selection).
hipError_t launch_block_scores(const SelectArgs &a, hipStream_t st);
// Bytes of the static device array that holds the pooled means for
// launch_select_scratch (which ignores a.qbar / a.kbarT and points them into
// that array); callers check 4 * nb * d * B * (Hq + Hkv) against it first.
constexpr size_t kSelectScratchBytes = (size_t)64 << 20;
hipError_t launch_select_scratch(SelectArgs a, hipStream_t st);
// ev: nullable, four events recorded before, between and after the three
// attention kernels
hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t st, hipEvent_t const *ev = nullptr);
// bytes of the attention workspace (partial state of every query row)
size_t attn_workspace_bytes(int B, int Hq, int N, int d);

}  // namespace thrift
