// Step 3 of the ThriftAttention path ("ThriftAttention: Selective Mixed
// Precision for Long-Context FP4 Attention", abstract): the selected
// query-key blocks are computed in FP16, the remaining ones in block-scaled
// 4-bit, and both paths are merged by one online softmax into one output.
//
// Work decomposition (gfx950, wave64):
//   * a workgroup owns one query block i (64 rows) of HPW query heads of one
//     GQA group and walks the valid key blocks j = 0..n_valid-1 in ascending
//     order -- the merge of the ascending FP16 and FP4 traversal lists;
//   * per key block it stages the MXFP4 tile (K codes/scales, V codes/scales)
//     when any of its heads has the block on its FP4 list and the FP16 tile
//     (K and channel-major V) when any head has it on its FP16 list, so GQA
//     heads share every K/V byte they read;
//   * a wave owns 32 query rows of one head and computes S^T = K Q^T with
//     32x32 MFMAs (FP16: v_mfma_f32_32x32x16_f16; FP4:
//     v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0 scales), then O^T += V^T P^T.
//
// Lane layout.  In a 32x32 MFMA result, lane l holds column l%32 and rows
// 8(r/4) + 4(l/32) + r%4 of accumulator register r.  K rows are fed to the
// A operand permuted so that lane l ends up holding, for query l%32, the 32
// keys 32(l/32) + 0..31 of the tile (register r of the first MFMA block is
// key 32(l/32) + r, of the second block key 32(l/32) + 16 + r).  One lane
// therefore holds exactly one aligned 32-key MX group of P for its query: the
// group's scale needs no cross-lane reduction, and the packed E2M1 codes are
// directly the B operand (lane l: column l%32, k = 32(l/32)..+31) of the FP4
// P.V product, whose A operand reads V's 32-token codes of the same group.
//
// Online softmax.  The running max is an integer M in log2 units
// (x = score * c, c = sm_scale * log2 e), so a change of M rescales the
// accumulator and row sum by an exact power of two, which leaves the MXFP4
// re-quantization of P (a per-group power-of-two scale) unchanged.  M is only
// raised when a tile's max exceeds it by more than kLazy, so p stays below
// 2^kLazy (fp16 P cannot overflow) and rescales are rare.
#include "thrift_internal.h"

namespace thrift {

constexpr float kLazy = 8.0f;

template <int D>
struct Tile {
  // FP4 stage
  static constexpr int K4 = 64 * D / 2, K4S = 64 * D / 32, V4 = D * 32, V4S = D * 2;
  static constexpr int FP4_BYTES = K4 + K4S + V4 + V4S;
  // FP16 stage
  static constexpr int K16 = 64 * D * 2, V16 = D * 64 * 2;
  static constexpr int FP16_BYTES = K16 + V16;
  static constexpr int STAGE = FP4_BYTES + FP16_BYTES;
  // offsets inside a stage
  static constexpr int oK4 = 0, oK4S = K4, oV4 = K4 + K4S, oV4S = K4 + K4S + V4;
  static constexpr int oK16 = FP4_BYTES, oV16 = FP4_BYTES + K16;
};

// Key (row of the 64-key tile) that A-operand row rho of MFMA block blk
// reads, so that the result lands in the lane layout described above.
__device__ __forceinline__ int permuted_key(int rho, int blk) {
  return 32 * ((rho >> 2) & 1) + 16 * blk + 4 * (rho >> 3) + (rho & 3);
}

template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) void attn_fwd_kernel(AttnArgs a) {
  using T = Tile<D>;
  constexpr int NT = 128 * HPW;                  // threads
  constexpr int C4 = T::FP4_BYTES / 16;          // 16-byte chunks of the FP4 stage
  constexpr int C16 = T::FP16_BYTES / 16;        // ... of the FP16 stage
  constexpr int R4 = (C4 + NT - 1) / NT;         // chunks per thread
  constexpr int R16 = (C16 + NT - 1) / NT;
  constexpr int KS16 = D / 16;                   // k-steps of the FP16 QK product
  constexpr int KS4 = D / 64;                    // k-steps of the FP4 QK product
  constexpr int CB = D / 32;                     // 32-channel blocks of O^T

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t *mask = (uint32_t *)(smem + 2 * T::STAGE);  // [HPW][kMaxBlocks/32] FP16-list bits

  const int nb = a.N / 64;
  const int group = a.Hq / a.Hkv;
  const int chunks = (group + HPW - 1) / HPW;
  const int per_i = a.B * a.Hkv * chunks;
  const int wi = blockIdx.x / per_i;
  int rem = blockIdx.x % per_i;
  const int i = a.causal ? nb - 1 - wi : wi;  // longest rows first
  const int b = rem / (a.Hkv * chunks);
  rem %= a.Hkv * chunks;
  const int g = rem / chunks, chunk = rem % chunks;
  const int nv = a.causal ? i + 1 : nb;
  const int nw = (nv + 31) / 32;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = wave >> 1, qhalf = wave & 1;
  const int hgrp = chunk * HPW + hl;
  const bool head_ok = hgrp < group;
  const int hq = g * group + (head_ok ? hgrp : 0);
  const int col = lane & 31, lh = lane >> 5;

  // ---- FP16-list bitmask of each head of the workgroup
  for (int w = tid; w < HPW * nw; w += NT) mask[(w / nw) * (kMaxBlocks / 32) + w % nw] = 0;
  __syncthreads();
  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  const int64_t roff = a.causal ? (int64_t)i * (i + 1) / 2 : (int64_t)i * nb;
  for (int h = 0; h < HPW; h++) {
    const int hg = chunk * HPW + h;
    if (hg >= group) break;
    const int64_t bh = (int64_t)b * a.Hq + g * group + hg;
    const int cnt = a.n16[bh * nb + i];
    const int32_t *l16 = a.idx + bh * per + roff;
    for (int e = tid; e < cnt; e += NT) {
      const int j = l16[e];
      if ((unsigned)j < (unsigned)nv) atomicOr(&mask[h * (kMaxBlocks / 32) + (j >> 5)], 1u << (j & 31));
    }
  }
  __syncthreads();
  const uint32_t head_bits = (chunk * HPW + HPW <= group) ? ((1u << HPW) - 1) : ((1u << (group - chunk * HPW)) - 1);
  auto fp16_heads = [&](int j) {
    uint32_t m = 0;
#pragma unroll
    for (int h = 0; h < HPW; h++) m |= ((mask[h * (kMaxBlocks / 32) + (j >> 5)] >> (j & 31)) & 1u) << h;
    return m & head_bits;
  };

  // ---- this wave's queries: Q16 and Q4 B-operands, held in registers
  const int64_t qrow = ((int64_t)b * a.Hq + hq) * a.N + 64 * (int64_t)i + 32 * qhalf + col;
  half8 qf16[KS16];
  int4v qf4[KS4];
  int qs4[KS4];
#pragma unroll
  for (int kk = 0; kk < KS16; kk++)
    qf16[kk] = __builtin_bit_cast(half8, *(const int4v *)(a.q16 + qrow * D + 16 * kk + 8 * lh));
#pragma unroll
  for (int kk = 0; kk < KS4; kk++) {
    qf4[kk] = *(const int4v *)(a.q4 + qrow * (D / 2) + 32 * kk + 16 * lh);
    qs4[kk] = a.q4s[qrow * (D / 32) + 2 * kk + lh];
  }

  // ---- K/V tile sources
  const int64_t kvh = (int64_t)b * a.Hkv + g;
  auto fp4_src = [&](int j, int c) -> const int4v * {
    const int off = 16 * c;
    if (off < T::oK4S) return (const int4v *)(a.k4 + (kvh * a.N + 64 * (int64_t)j) * (D / 2) + off);
    if (off < T::oV4) return (const int4v *)(a.k4s + (kvh * a.N + 64 * (int64_t)j) * (D / 32) + (off - T::oK4S));
    if (off < T::oV4S) return (const int4v *)(a.v4 + (kvh * nb + j) * (int64_t)(32 * D) + (off - T::oV4));
    return (const int4v *)(a.v4s + (kvh * nb + j) * (int64_t)(2 * D) + (off - T::oV4S));
  };
  auto fp16_src = [&](int j, int c) -> const int4v * {
    const int off = 16 * c;
    if (off < T::K16) return (const int4v *)((const uint8_t *)a.k16 + (kvh * a.N + 64 * (int64_t)j) * (2 * D) + off);
    return (const int4v *)((const uint8_t *)a.v16 + (kvh * nb + j) * (int64_t)(128 * D) + (off - T::K16));
  };
  int4v pre4[R4], pre16[R16];
  auto prefetch = [&](int j, uint32_t h16) {
    const bool need16 = h16 != 0, need4 = h16 != head_bits;
    if (need4) {
#pragma unroll
      for (int r = 0; r < R4; r++) {
        const int c = tid + r * NT;
        if (c < C4) pre4[r] = *fp4_src(j, c);
      }
    }
    if (need16) {
#pragma unroll
      for (int r = 0; r < R16; r++) {
        const int c = tid + r * NT;
        if (c < C16) pre16[r] = *fp16_src(j, c);
      }
    }
  };
  auto commit = [&](uint8_t *st, uint32_t h16) {
    const bool need16 = h16 != 0, need4 = h16 != head_bits;
    if (need4) {
#pragma unroll
      for (int r = 0; r < R4; r++) {
        const int c = tid + r * NT;
        if (c < C4) *(int4v *)(st + 16 * c) = pre4[r];
      }
    }
    if (need16) {
#pragma unroll
      for (int r = 0; r < R16; r++) {
        const int c = tid + r * NT;
        if (c < C16) *(int4v *)(st + T::FP4_BYTES + 16 * c) = pre16[r];
      }
    }
  };

  // ---- softmax state and accumulators
  float16v acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[cb][r] = 0.0f;
  float M = -INFINITY, l_part = 0.0f;
  const float c = a.c;
  const int qpos = 32 * qhalf + col;  // query row inside the block

  uint32_t h16_cur = fp16_heads(0);
  prefetch(0, h16_cur);
  commit(smem, h16_cur);
  __syncthreads();

  for (int j = 0; j < nv; j++) {
    const uint8_t *st = smem + (j & 1) * T::STAGE;
    uint32_t h16_next = 0;
    if (j + 1 < nv) {
      h16_next = fp16_heads(j + 1);
      prefetch(j + 1, h16_next);
    }
    if (head_ok) {
      const bool use16 = (h16_cur >> hl) & 1u;
      const bool diag = a.causal && (j == i);
      // S^T = K Q^T for the two 32-key halves of the permuted tile
      float16v s[2];
#pragma unroll
      for (int blk = 0; blk < 2; blk++) {
#pragma unroll
        for (int r = 0; r < 16; r++) s[blk][r] = 0.0f;
        const int key = permuted_key(col, blk);
        if (use16) {
          const uint8_t *krow = st + T::oK16 + key * (2 * D);
#pragma unroll
          for (int kk = 0; kk < KS16; kk++) {
            half8 kf = __builtin_bit_cast(half8, *(const int4v *)(krow + 2 * (16 * kk + 8 * lh)));
            s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf16[kk], s[blk], 0, 0, 0);
          }
        } else {
          const uint8_t *krow = st + T::oK4 + key * (D / 2);
          const uint8_t *ksc = st + T::oK4S + key * (D / 32);
#pragma unroll
          for (int kk = 0; kk < KS4; kk++) {
            int4v kf = *(const int4v *)(krow + 32 * kk + 16 * lh);
            int8v ka = {kf[0], kf[1], kf[2], kf[3], 0, 0, 0, 0};
            int8v qb = {qf4[kk][0], qf4[kk][1], qf4[kk][2], qf4[kk][3], 0, 0, 0, 0};
            s[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qb, s[blk], 4, 4, 0, (int)ksc[2 * kk + lh], 0,
                                                                      qs4[kk]);
          }
        }
      }
      // causal mask: key 32*lh + idx of this lane vs query qpos
      if (diag) {
#pragma unroll
        for (int blk = 0; blk < 2; blk++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            if (32 * lh + 16 * blk + r > qpos) s[blk][r] = -INFINITY;
      }
      // row max over this lane's 32 keys, then over the partner lane's
      float smax = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; blk++)
#pragma unroll
        for (int r = 0; r < 16; r++) smax = fmaxf(smax, s[blk][r]);
      const float lane_max = smax;
      smax = fmaxf(smax, __shfl_xor(smax, 32));
      const float mt = ceilf(smax * c);  // integer candidate max (log2 units)
      const bool raise = mt > M + kLazy || M == -INFINITY;
      if (__any(raise)) {
        if (raise) {
          const float sc = (M == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(M - mt));
          l_part *= sc;
#pragma unroll
          for (int cb = 0; cb < CB; cb++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[cb][r] *= sc;
          M = mt;
        }
      }
      const float negM = -M;
      // p = 2^(x - M); masked keys give 2^-inf = 0
      float lsum = 0.0f;
#pragma unroll
      for (int blk = 0; blk < 2; blk++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[blk][r], c, negM));
          s[blk][r] = p;
          lsum += p;
        }
      l_part += lsum;
      if (use16) {
        // P in fp16; MFMA u consumes keys 32*lh + 8u + 0..7 of this lane
        half8 pb[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
          for (int t = 0; t < 8; t++) pb[u][t] = (_Float16)s[u >> 1][8 * (u & 1) + t];
        const uint8_t *vt = st + T::oV16;
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
          const int ch = 32 * cb + col;
#pragma unroll
          for (int u = 0; u < 4; u++) {
            half8 vf = __builtin_bit_cast(half8, *(const int4v *)(vt + ch * 128 + 2 * (32 * lh + 8 * u)));
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pb[u], acc[cb], 0, 0, 0);
          }
        }
      } else {
        // P re-quantized to MXFP4: this lane's 32 values are one aligned group
        const float amax = __builtin_amdgcn_exp2f(fmaf(lane_max, c, negM));
        const int psb = mx_scale_byte(amax);
        const float div = mx_scale_divisor(psb);
        uint32_t pw[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const int blk = w >> 1, r0 = 8 * (w & 1);
          THRIFT_CVT_FP4(pw[w], s[blk][r0 + 0], s[blk][r0 + 1], div, 0);
          THRIFT_CVT_FP4(pw[w], s[blk][r0 + 2], s[blk][r0 + 3], div, 1);
          THRIFT_CVT_FP4(pw[w], s[blk][r0 + 4], s[blk][r0 + 5], div, 2);
          THRIFT_CVT_FP4(pw[w], s[blk][r0 + 6], s[blk][r0 + 7], div, 3);
        }
        int8v pbv = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], 0, 0, 0, 0};
        const uint8_t *vt = st + T::oV4;
        const uint8_t *vs = st + T::oV4S;
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
          const int ch = 32 * cb + col;
          int4v vf = *(const int4v *)(vt + ch * 32 + 16 * lh);
          int8v va = {vf[0], vf[1], vf[2], vf[3], 0, 0, 0, 0};
          acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pbv, acc[cb], 4, 4, 0, (int)vs[ch * 2 + lh], 0,
                                                                     psb);
        }
      }
    }
    if (j + 1 < nv) commit(smem + ((j + 1) & 1) * T::STAGE, h16_next);
    h16_cur = h16_next;
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = (M + log2 l) ln 2
  if (!head_ok) return;
  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l;
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const int ch = 32 * cb + 8 * q4 + 4 * lh;  // rows 8(r/4) + 4(lane/32) + r%4 of block cb
      float4v o = {acc[cb][4 * q4 + 0] * inv, acc[cb][4 * q4 + 1] * inv, acc[cb][4 * q4 + 2] * inv,
                   acc[cb][4 * q4 + 3] * inv};
      if (a.out_dtype == 2) {
        *(float4v *)((float *)a.out + qrow * D + ch) = o;
      } else if (a.out_dtype == 0) {
        _Float16 *op = (_Float16 *)a.out + qrow * D + ch;
        for (int e = 0; e < 4; e++) op[e] = (_Float16)o[e];
      } else {
        uint16_t *op = (uint16_t *)a.out + qrow * D + ch;
        for (int e = 0; e < 4; e++) {
          uint32_t u = __float_as_uint(o[e]);
          u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even (finite values)
          op[e] = (uint16_t)(u >> 16);
        }
      }
    }
  }
  if (a.lse && lh == 0) a.lse[qrow] = (M + __log2f(l)) * 0.69314718055994530942f;
}

template <int D, int HPW>
static hipError_t launch_one(const AttnArgs &a, hipStream_t st) {
  using T = Tile<D>;
  const int group = a.Hq / a.Hkv;
  const int chunks = (group + HPW - 1) / HPW;
  const size_t lds = 2 * (size_t)T::STAGE + (size_t)HPW * (kMaxBlocks / 32) * 4;
  hipError_t e = hipFuncSetAttribute((const void *)attn_fwd_kernel<D, HPW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((int64_t)(a.N / 64) * a.B * a.Hkv * chunks);
  hipLaunchKernelGGL((attn_fwd_kernel<D, HPW>), dim3(grid), dim3(128 * HPW), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t st) {
  const int group = a.Hq / a.Hkv;
  const int hpw = group >= 4 ? 4 : (group >= 2 ? 2 : 1);
  if (a.d == 128) {
    if (hpw == 4) return launch_one<128, 4>(a, st);
    if (hpw == 2) return launch_one<128, 2>(a, st);
    return launch_one<128, 1>(a, st);
  }
  if (hpw == 4) return launch_one<64, 4>(a, st);
  if (hpw == 2) return launch_one<64, 2>(a, st);
  return launch_one<64, 1>(a, st);
}

}  // namespace thrift
