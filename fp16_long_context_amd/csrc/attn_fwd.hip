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
// Largest p an FP4-only tile may reach against the running max (2^64).
// With |v| <= 2^16 and at most 2^19 keys, acc stays below 2^(64 + 16 + 19)
// = 2^99 and P's scale byte at most 127 + 64 - 2 = 189.
constexpr float kMaxP = 0x1p64f;

template <int D, int HPW>
struct Tile {
  // FP4 stage
  static constexpr int K4 = 64 * D / 2, K4S = 64 * D / 32, V4 = D * 32, V4S = D * 2;
  static constexpr int FP4_BYTES = K4 + K4S + V4 + V4S;
  // FP16 stage
  static constexpr int K16 = 64 * D * 2, V16 = D * 64 * 2;
  static constexpr int FP16_BYTES = K16 + V16;
  static constexpr int STAGE = FP4_BYTES + FP16_BYTES;
  // offsets inside a stage: codes first (whole 1 KB groups per region), then
  // the K and V scale bytes
  static constexpr int oK4 = 0, oV4 = K4, oK4S = K4 + V4, oV4S = K4 + V4 + K4S;
  static constexpr int G4 = (K4 + V4) / 1024;    // 64-chunk groups of FP4 codes
  static constexpr int SC4 = (K4S + V4S) / 16;   // 16-byte chunks of FP4 scales
  static constexpr int G16 = (K16 + V16) / 1024; // 64-chunk groups of the FP16 stage
  // the FP4-only walk uses a 3-slot ring of FP4 stages in the same memory
  static constexpr int RING = FP4_BYTES;
  static constexpr int oK16 = FP4_BYTES, oV16 = FP4_BYTES + K16;
  // after the two stages: the workgroup's Q16 rows ([HPW*64][D] halves,
  // 16-byte chunks XOR-swizzled by row) and the FP16-list bitmasks
  static constexpr int oQ16 = 2 * STAGE;
  static constexpr int Q16_BYTES = HPW * 64 * D * 2;
  static constexpr int oMASK = oQ16 + Q16_BYTES;
  static constexpr int oUMASK = oMASK + HPW * (kMaxBlocks / 32) * 4;  // union of the heads' FP16 lists
  static constexpr int LDS = oUMASK + (kMaxBlocks / 32) * 4;
};

// LDS layouts of the staged tiles are XOR-swizzled in 16-byte chunks so that
// the MFMA operand reads (32 permuted key rows, or 32 consecutive channel
// rows, at the same logical chunk) spread over all LDS banks.  Physical chunk
// = logical chunk ^ swz(row).  The loader applies the same map to the source
// address, so the direct global->LDS copy stays a plain per-lane transfer.
// The maps keep every group of 8 lanes (128 bytes) and of 16 lanes (256
// bytes) of an operand read on distinct bank slots.
template <int D>
__device__ __forceinline__ int swz_k4(int key) {  // K4 rows: D/32 chunks
  if (D == 128) return (((key >> 1) ^ (key >> 2)) & 1) | (((key >> 5) & 1) << 1);
  return (key >> 5) & 1;
}
template <int D>
__device__ __forceinline__ int swz_k16(int key) {  // K16 rows: D/8 chunks
  if (D == 128) return (key & 3) | (((key >> 5) & 1) << 2) | (((key >> 2) & 1) << 3);
  return ((key >> 1) & 1) | (((key >> 2) & 1) << 1) | (((key >> 5) & 1) << 2);
}
__device__ __forceinline__ int swz_v16(int ch) { return (ch ^ (ch >> 3)) & 7; }       // V16 rows: 8 chunks
__device__ __forceinline__ int swz_v4(int ch) { return ((ch >> 2) ^ (ch >> 3)) & 1; }  // V4 rows: 2 chunks

// Key (row of the 64-key tile) that A-operand row rho of MFMA block blk
// reads, so that the result lands in the lane layout described above.
__device__ __forceinline__ int permuted_key(int rho, int blk) {
  return 32 * ((rho >> 2) & 1) + 16 * blk + 4 * (rho >> 3) + (rho & 3);
}

// 16 bytes per lane from global memory straight into LDS at lds_wave_base +
// 16 * lane (lds_wave_base must be the same for the whole wave).
__device__ __forceinline__ void load_to_lds(const void *g, uint8_t *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}

// Wait until this wave's outstanding vector-memory loads (including the
// direct-to-LDS ones) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The value x of lane l^32 (v_permlane32_swap exchanges the wave's halves).
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Largest of this lane's 32 scores (v_max3 chain).
__device__ __forceinline__ float lane_max32(const float16v (&s)[2]) {
  float m[4] = {fmaxf(s[0][0], s[0][1]), fmaxf(s[0][8], s[0][9]), fmaxf(s[1][0], s[1][1]), fmaxf(s[1][8], s[1][9])};
#pragma unroll
  for (int r = 2; r < 8; r += 2) {
    m[0] = fmaxf(fmaxf(m[0], s[0][r]), s[0][r + 1]);
    m[1] = fmaxf(fmaxf(m[1], s[0][8 + r]), s[0][9 + r]);
    m[2] = fmaxf(fmaxf(m[2], s[1][r]), s[1][r + 1]);
    m[3] = fmaxf(fmaxf(m[3], s[1][8 + r]), s[1][9 + r]);
  }
  return fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
}

// Online-softmax step on one 32-query x 64-key score tile held as s[2]
// (this lane: query col, keys 32*lh + 0..31).  Applies the causal mask on
// the diagonal tile, raises the integer running max when needed (rescaling
// acc and the row sum by an exact power of two), replaces s by
// p = 2^(s*c - M) and adds the lane's p to l_part.  Returns the lane's
// largest raw score (-inf if all masked).
template <int CB, bool MASK>
__device__ __forceinline__ float softmax_step(float16v (&s)[2], float16v (&acc)[CB], float &M, float &l_part,
                                              const float c, const int lh, const int qpos) {
  if (MASK) {
#pragma unroll
    for (int blk = 0; blk < 2; blk++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (32 * lh + 16 * blk + r > qpos) s[blk][r] = -INFINITY;
  }
  const float lane_max = lane_max32(s);
  const float row_max = fmaxf(lane_max, other_half(lane_max));
  const float mt = ceilf(row_max * c);  // integer candidate max (log2 units)
  const bool raise = (mt > M + kLazy) || (M == -INFINITY);
  if (__ballot(raise)) {  // wave-uniform; lanes that keep their max scale by 1
    const float sc = raise ? ((M == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(M - mt))) : 1.0f;
    M = raise ? mt : M;
    l_part *= sc;
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[cb][r] *= sc;
  }
  const float negM = -M;
  float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s[0][r] = __builtin_amdgcn_exp2f(fmaf(s[0][r], c, negM));
    s[1][r] = __builtin_amdgcn_exp2f(fmaf(s[1][r], c, negM));
    l0 += s[0][r];
    l1 += s[1][r];
  }
  l_part += l0 + l1;
  return lane_max;
}

// K operands (MXFP4 codes and scale bytes) of an FP4 tile's QK product.
template <int D, int HPW>
__device__ __forceinline__ void fp4_kops(const uint8_t *st, const int col, const int lh, int4v (&ka)[2][D / 64],
                                         int (&ks)[2][D / 64]) {
  using T = Tile<D, HPW>;
#pragma unroll
  for (int blk = 0; blk < 2; blk++) {
    const int key = permuted_key(col, blk);
#pragma unroll
    for (int kk = 0; kk < D / 64; kk++) {
      ka[blk][kk] = *(const int4v *)(st + T::oK4 + key * (D / 2) + 16 * ((2 * kk + lh) ^ swz_k4<D>(key)));
      ks[blk][kk] = st[T::oK4S + key * (D / 32) + 2 * kk + lh];
    }
  }
}

// S^T = K4 Q4^T for the two 32-key halves of the permuted tile.
template <int D>
__device__ __forceinline__ void fp4_qk_mfma(const int4v (&ka)[2][D / 64], const int (&ks)[2][D / 64],
                                            const int4v (&qf4)[D / 64], const int (&qs4)[D / 64],
                                            float16v (&s)[2]) {
#pragma unroll
  for (int blk = 0; blk < 2; blk++) {
#pragma unroll
    for (int r = 0; r < 16; r++) s[blk][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 64; kk++) {
      int8v a8 = {ka[blk][kk][0], ka[blk][kk][1], ka[blk][kk][2], ka[blk][kk][3], 0, 0, 0, 0};
      int8v b8 = {qf4[kk][0], qf4[kk][1], qf4[kk][2], qf4[kk][3], 0, 0, 0, 0};
      s[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, s[blk], 4, 4, 0, ks[blk][kk], 0, qs4[kk]);
    }
  }
}

// S^T = K4 Q4^T of an FP4 tile (operand reads + MFMAs).
template <int D, int HPW>
__device__ __forceinline__ void fp4_qk(const uint8_t *st, const int4v (&qf4)[D / 64], const int (&qs4)[D / 64],
                                       const int col, const int lh, float16v (&s)[2]) {
  int4v ka[2][D / 64];
  int ks[2][D / 64];
  fp4_kops<D, HPW>(st, col, lh, ka, ks);
  fp4_qk_mfma<D>(ka, ks, qf4, qs4, s);
}

// The V operands (MXFP4 codes and scales) of an FP4 tile's P.V product.
template <int D, int HPW>
__device__ __forceinline__ void fp4_vops(const uint8_t *st, const int col, const int lh, int4v (&va)[D / 32],
                                         int (&vs)[D / 32]) {
  using T = Tile<D, HPW>;
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) {
    const int ch = 32 * cb + col;
    va[cb] = *(const int4v *)(st + T::oV4 + ch * 32 + 16 * (lh ^ swz_v4(ch)));
    vs[cb] = st[T::oV4S + ch * 2 + lh];
  }
}

// FP4 tile, first half: S^T (masked on the diagonal) and the V operands
// (read here so their LDS latency hides under the softmax).
template <int D, int HPW, bool MASK>
__device__ __forceinline__ void fp4_scores(const uint8_t *st, const int4v (&qf4)[D / 64], const int (&qs4)[D / 64],
                                           const int col, const int lh, const int qpos, float16v (&s)[2],
                                           int4v (&va)[D / 32], int (&vs)[D / 32]) {
  fp4_qk<D, HPW>(st, qf4, qs4, col, lh, s);
  fp4_vops<D, HPW>(st, col, lh, va, vs);
  if (MASK) {
#pragma unroll
    for (int blk = 0; blk < 2; blk++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (32 * lh + 16 * blk + r > qpos) s[blk][r] = -INFINITY;
  }
}

// FP4 tile, second half: p (this lane's 32 values, one aligned 32-key group,
// relative to the max the exponent used) re-quantized to MXFP4, and
// O^T += V^T P^T.  `shift` is an extra power of two folded into P's E8M0
// scale (the group's contribution is exactly 2^shift times its codes).
template <int CB>
__device__ __forceinline__ void fp4_pv(const float16v (&s)[2], const float amax, const int shift,
                                       const int4v (&va)[CB], const int (&vs)[CB], float16v (&acc)[CB]) {
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
  int8v pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], 0, 0, 0, 0};
  const int pscale = psb + shift;
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    int8v a8 = {va[cb][0], va[cb][1], va[cb][2], va[cb][3], 0, 0, 0, 0};
    acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, pb, acc[cb], 4, 4, 0, vs[cb], 0, pscale);
  }
}

// One FP4 tile (general walk): the running max may rise, rescaling acc.
template <int D, int HPW, bool MASK>
__device__ __forceinline__ void tile_fp4(const uint8_t *st, const int4v (&qf4)[D / 64], const int (&qs4)[D / 64],
                                         float16v (&acc)[D / 32], float &M, float &l_part, const float c,
                                         const int col, const int lh, const int qpos) {
  constexpr int CB = D / 32;
  float16v s[2];
  int4v va[CB];
  int vs[CB];
  fp4_scores<D, HPW, MASK>(st, qf4, qs4, col, lh, qpos, s, va, vs);
  const float lane_max = softmax_step<CB, false>(s, acc, M, l_part, c, lh, qpos);
  fp4_pv<CB>(s, __builtin_amdgcn_exp2f(fmaf(lane_max, c, -M)), 0, va, vs, acc);
}

// Softmax and P.V of one FP4-only tile whose scores s are already computed.
// The running max M is final for this walk (it was set by the FP16-union
// walk and the diagonal): p = 2^(s*c - M) is taken directly, so no step of
// the exponentials waits on this tile's max.  P's group scale comes from the
// largest p of the lane's 32-key group (the MXFP4 rule's amax, taken after
// the exponentials); a group with amax above kMaxP (or infinite) sets
// `overflow`, and the work item is then redone with the rescaling walk.
template <int CB>
__device__ __forceinline__ void fp4_fixed_rest(float16v (&s)[2], const int4v (&va)[CB], const int (&vs)[CB],
                                               float16v (&acc)[CB], const float M, float &l_part, bool &overflow,
                                               const float c) {
  const float negM = -M;
  float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s[0][r] = __builtin_amdgcn_exp2f(fmaf(s[0][r], c, negM));
    s[1][r] = __builtin_amdgcn_exp2f(fmaf(s[1][r], c, negM));
    l0 += s[0][r];
    l1 += s[1][r];
  }
  l_part += l0 + l1;
  const float amax = lane_max32(s);
  overflow = overflow || !(amax <= kMaxP);
  fp4_pv<CB>(s, amax, 0, va, vs, acc);
}

// One FP16 tile for one wave: S^T from FP16 K and Q, P rounded to fp16,
// O^T += V^T P^T with FP16 V.  qrow16 points at this lane's Q16 row in LDS.
template <int D, int HPW, bool MASK>
__device__ __forceinline__ void tile_fp16(const uint8_t *st, const uint8_t *qrow16, float16v (&acc)[D / 32],
                                          float &M, float &l_part, const float c, const int col, const int lh,
                                          const int qpos) {
  using T = Tile<D, HPW>;
  constexpr int KS = D / 16, CB = D / 32, CPR = D / 8;  // k-steps, channel blocks, 16-byte chunks per row
  float16v s[2];
#pragma unroll
  for (int blk = 0; blk < 2; blk++)
#pragma unroll
    for (int r = 0; r < 16; r++) s[blk][r] = 0.0f;
  const int key0 = permuted_key(col, 0), key1 = permuted_key(col, 1);
  const uint8_t *k0 = st + T::oK16 + key0 * (2 * D);
  const uint8_t *k1 = st + T::oK16 + key1 * (2 * D);
  const int sw0 = swz_k16<D>(key0), sw1 = swz_k16<D>(key1);
#pragma unroll
  for (int kk = 0; kk < KS; kk += 2) {
    half8 qb[2], a0[2], a1[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int chunk = 2 * (kk + u) + lh;
      qb[u] = __builtin_bit_cast(half8, *(const int4v *)(qrow16 + 16 * (chunk ^ (col & (CPR - 1)))));
      a0[u] = __builtin_bit_cast(half8, *(const int4v *)(k0 + 16 * (chunk ^ sw0)));
      a1[u] = __builtin_bit_cast(half8, *(const int4v *)(k1 + 16 * (chunk ^ sw1)));
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[u], qb[u], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[u], qb[u], s[1], 0, 0, 0);
    }
  }
  softmax_step<CB, MASK>(s, acc, M, l_part, c, lh, qpos);
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
    half8 vf[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
      vf[u] = __builtin_bit_cast(half8, *(const int4v *)(vt + ch * 128 + 16 * ((4 * lh + u) ^ swz_v16(ch))));
#pragma unroll
    for (int u = 0; u < 4; u++) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[u], pb[u], acc[cb], 0, 0, 0);
  }
}

template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) void attn_fwd_kernel(AttnArgs a) {
  using T = Tile<D, HPW>;
  constexpr int NT = 128 * HPW;                  // threads
  constexpr int KS4 = D / 64;                    // k-steps of the FP4 QK product
  constexpr int CB = D / 32;                     // 32-channel blocks of O^T
  constexpr int CPR = D / 8;                     // 16-byte chunks per Q16 row

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t *mask = (uint32_t *)(smem + T::oMASK);  // [HPW][kMaxBlocks/32] FP16-list bits

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
  // ---- this wave's 32 query rows: Q16 into LDS (swizzled), Q4 into registers
  const int64_t qrow0 = ((int64_t)b * a.Hq + hq) * a.N + 64 * (int64_t)i + 32 * qhalf;
  uint8_t *q16w = smem + T::oQ16 + (size_t)wave * 32 * D * 2;
#pragma unroll
  for (int it = 0; it < CPR / 2; it++) {  // 32 rows x CPR chunks over 64 lanes
    const int e = lane + 64 * it, row = e / CPR, ch = e % CPR;
    const int4v v = *(const int4v *)(a.q16 + (qrow0 + row) * D + 8 * ch);
    *(int4v *)(q16w + row * (2 * D) + 16 * (ch ^ (row & (CPR - 1)))) = v;
  }
  const int64_t qrow = qrow0 + col;
  int4v qf4[KS4];
  int qs4[KS4];
#pragma unroll
  for (int kk = 0; kk < KS4; kk++) {
    qf4[kk] = *(const int4v *)(a.q4 + qrow * (D / 2) + 32 * kk + 16 * lh);
    qs4[kk] = a.q4s[qrow * (D / 32) + 2 * kk + lh];
  }
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
    return (uint32_t)__builtin_amdgcn_readfirstlane(m & head_bits);
  };

  // ---- K/V tile loads: direct global -> LDS copies (global_load_lds_dwordx4;
  // lane L of a wave writes its 16 bytes at the wave-uniform LDS base + 16 L).
  // Each wave copies whole 1 KB groups of one region, so the region choice is
  // scalar and the source address is a scalar base plus a per-lane offset
  // (with the chunk swizzle of the region).  The caller waits (vmcnt) before
  // the barrier that publishes the stage.
  constexpr int NWAVES = 2 * HPW;
  const int64_t kvh = (int64_t)b * a.Hkv + g;
  const uint8_t *k4b = a.k4 + kvh * a.N * (D / 2), *k4sb = a.k4s + kvh * a.N * (D / 32);
  const uint8_t *v4b = a.v4 + kvh * nb * (int64_t)(32 * D), *v4sb = a.v4s + kvh * nb * (int64_t)(2 * D);
  const uint8_t *k16b = (const uint8_t *)a.k16 + kvh * a.N * (2 * D);
  const uint8_t *v16b = (const uint8_t *)a.v16 + kvh * nb * (int64_t)(128 * D);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // FP4-only walk: this wave's code groups t = wave_u + g * NWAVES (< G4)
  // have fixed per-lane offsets inside a tile; per tile only the scalar base
  // moves (j times the array's per-block stride).
  constexpr int NG4 = (T::G4 + NWAVES - 1) / NWAVES;
  uint32_t goff[NG4];
#pragma unroll
  for (int g = 0; g < NG4; g++) {
    const int t = wave_u + g * NWAVES;
    if (t < T::K4 / 1024) {
      const int off = 1024 * t + 16 * lane, key = off / (D / 2), pch = (off % (D / 2)) / 16;
      goff[g] = key * (D / 2) + 16 * (pch ^ swz_k4<D>(key));
    } else {
      const int o = 1024 * (t - T::K4 / 1024) + 16 * lane, ch = o / 32, pch = (o % 32) / 16;
      goff[g] = ch * 32 + 16 * (pch ^ swz_v4(ch));
    }
  }
  auto issue_fp4 = [&](uint8_t *st, int j) {
#pragma unroll
    for (int g = 0; g < NG4; g++) {
      const int t = wave_u + g * NWAVES;
      if (t < T::G4) {
        const uint8_t *base = (t < T::K4 / 1024) ? k4b + (int64_t)j * (64 * D / 2) : v4b + (int64_t)j * (32 * D);
        load_to_lds(base + goff[g], st + 1024 * t);
      }
    }
    if (wave_u == NWAVES - 1) {
      if (lane < T::K4S / 16)
        load_to_lds(k4sb + (int64_t)j * (64 * D / 32) + 16 * lane, st + T::oK4S);
      else if (lane < T::SC4)
        load_to_lds(v4sb + (int64_t)j * (2 * D) + 16 * (lane - T::K4S / 16), st + T::oK4S);
    }
  };
  auto issue_loads = [&](uint8_t *st, int j, uint32_t h16) {
    if (h16 != head_bits) {
      for (int t = wave_u; t < T::G4; t += NWAVES) {
        const uint8_t *src;
        if (t < T::K4 / 1024) {
          const int off = 1024 * t + 16 * lane, key = off / (D / 2), pch = (off % (D / 2)) / 16;
          src = k4b + (int64_t)j * (64 * D / 2) + key * (D / 2) + 16 * (pch ^ swz_k4<D>(key));
        } else {
          const int o = 1024 * (t - T::K4 / 1024) + 16 * lane, ch = o / 32, pch = (o % 32) / 16;
          src = v4b + (int64_t)j * (32 * D) + ch * 32 + 16 * (pch ^ swz_v4(ch));
        }
        load_to_lds(src, st + 1024 * t);
      }
      if (wave_u == NWAVES - 1 && lane < T::SC4) {
        const uint8_t *src = lane < T::K4S / 16 ? k4sb + (int64_t)j * (64 * D / 32) + 16 * lane
                                                : v4sb + (int64_t)j * (2 * D) + 16 * (lane - T::K4S / 16);
        load_to_lds(src, st + T::oK4S);
      }
    }
    if (h16 != 0) {
      for (int t = wave_u; t < T::G16; t += NWAVES) {
        const uint8_t *src;
        if (t < T::K16 / 1024) {
          const int off = 1024 * t + 16 * lane, key = off / (2 * D), pch = (off % (2 * D)) / 16;
          src = k16b + (int64_t)j * (64 * 2 * D) + key * (2 * D) + 16 * (pch ^ swz_k16<D>(key));
        } else {
          const int o = 1024 * (t - T::K16 / 1024) + 16 * lane, ch = o / 128, pch = (o % 128) / 16;
          src = v16b + (int64_t)j * (128 * D) + ch * 128 + 16 * (pch ^ swz_v16(ch));
        }
        load_to_lds(src, st + T::oK16 + 1024 * t);
      }
    }
  };

  const float c = a.c;
  const int qpos = 32 * qhalf + col;  // query row inside the block
  const uint8_t *qrow16 = q16w + col * (2 * D);

  // ---- traversal.  Phase 1 walks the union of the heads' FP16 lists (all
  // FP16 tiles, the first and the diagonal block), where the row max is
  // almost always reached; phase 2 walks the blocks every head has on its
  // FP4 list, with the accumulator left unscaled (fp4_fixed_rest).  Both
  // walks are ascending and prefetch ahead of the tile being computed.
  uint32_t *umask = (uint32_t *)(smem + T::oUMASK);
  for (int w = tid; w < nw; w += NT) {
    uint32_t u = 0;
#pragma unroll
    for (int h = 0; h < HPW; h++)
      if ((head_bits >> h) & 1u) u |= mask[h * (kMaxBlocks / 32) + w];
    umask[w] = u;
  }
  __syncthreads();
  // Causal rows end at the diagonal block, which takes the masked bodies and
  // is handled on its own between the two walks (so neither walk's loop body
  // branches on it).
  const int jend = a.causal ? nv - 1 : nv;  // walks cover [0, jend)
  auto next_tile = [&](int j, bool in16) -> int {  // smallest j' >= j of the walk's set below jend, else nv
    for (int w = j >> 5; w < nw; w++) {
      uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane(umask[w]);
      if (!in16) m = ~m;
      if (w == (j >> 5)) m &= ~0u << (j & 31);
      if (m) {
        const int jj = 32 * w + __builtin_ctz(m);
        return jj < jend ? jj : nv;
      }
    }
    return nv;
  };

  // Pass 0 normally finishes the work item.  If an FP4-only tile reached
  // p > kMaxP in some row (a key far above every FP16-union block),
  // the workgroup redoes the item as pass 1, whose FP4-only walk raises the
  // running max as needed (the general tile body).
  for (int pass = 0; pass < 2; pass++) {
    float16v acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[cb][r] = 0.0f;
    float M = -INFINITY, l_part = 0.0f;
    bool overflow = false;

    // tile order: phase-1 tiles, the diagonal (causal), phase-2 tiles
    int j = next_tile(0, true);
    if (j >= nv) j = a.causal ? nv - 1 : nv;
    uint32_t h16_cur = (j < nv) ? fp16_heads(j) : 0u;
    int par = 0;
    if (j < nv) issue_loads(smem, j, h16_cur);
    wait_vmem();
    __syncthreads();
    // phase 1 (below the diagonal)
    while (j < jend) {
      int jn = next_tile(j + 1, true);
      if (jn >= nv) jn = a.causal ? nv - 1 : nv;
      const uint32_t h16_next = (jn < nv) ? fp16_heads(jn) : 0u;
      if (jn < nv) issue_loads(smem + (par ^ 1) * T::STAGE, jn, h16_next);
      const uint8_t *st = smem + par * T::STAGE;
      if (head_ok) {
        if ((h16_cur >> hl) & 1u)
          tile_fp16<D, HPW, false>(st, qrow16, acc, M, l_part, c, col, lh, qpos);
        else
          tile_fp4<D, HPW, false>(st, qf4, qs4, acc, M, l_part, c, col, lh, qpos);
      }
      wait_vmem();
      __syncthreads();
      par ^= 1;
      j = jn;
      h16_cur = h16_next;
    }
    // the diagonal tile (causal)
    if (j < nv) {
      const uint8_t *st = smem + par * T::STAGE;
      if (head_ok) {
        if ((h16_cur >> hl) & 1u)
          tile_fp16<D, HPW, true>(st, qrow16, acc, M, l_part, c, col, lh, qpos);
        else
          tile_fp4<D, HPW, true>(st, qf4, qs4, acc, M, l_part, c, col, lh, qpos);
      }
      __syncthreads();
    }
    // Phase 2 (below the diagonal): every head computes these in FP4.  A
    // 3-slot ring of FP4 stages (reusing the stage memory): while tile k is
    // in softmax/P.V, the QK MFMAs of tile k+1 are already issued and tile
    // k+2 is loading.  The loop is unrolled over the ring period so every LDS
    // offset is a constant.  The walk reads the complement of the FP16 union
    // one 32-block word at a time, kept in a scalar register.
    {
      int it_w = 0;
      uint32_t it_bits = 0;  // unvisited FP4-only blocks of word it_w
      auto it_load = [&](int w) {
        it_w = w;
        uint32_t m = (w < nw) ? ~(uint32_t)__builtin_amdgcn_readfirstlane(umask[w]) : 0u;
        const int hi = jend - 32 * w;  // blocks of this word below jend
        if (hi < 32) m &= hi > 0 ? ((1u << hi) - 1u) : 0u;
        it_bits = m;
      };
      auto it_next = [&]() -> int {  // next FP4-only block in ascending order, else nv
        while (it_bits == 0) {
          if (it_w + 1 >= nw) return nv;
          it_load(it_w + 1);
        }
        const int jj = 32 * it_w + __builtin_ctz(it_bits);
        it_bits &= it_bits - 1;
        return jj;
      };
      it_load(0);
      int jc = it_next();
      int jn = (jc < nv) ? it_next() : nv;
      if (jc < nv) issue_fp4(smem, jc);
      if (jn < nv) issue_fp4(smem + T::RING, jn);
      wait_vmem();
      __syncthreads();
      float16v sa[2], sb[2];
      if (pass == 0 && jc < nv && head_ok) {
        fp4_qk<D, HPW>(smem, qf4, qs4, col, lh, sa);
        // a row with no earlier tile takes its M from this first tile
        const float lm = lane_max32(sa);
        const float mt = ceilf(fmaxf(lm, other_half(lm)) * c);
        M = (M == -INFINITY) ? mt : M;
      }
      auto step = [&](const int cur, const int nxt, const int ldslot, float16v (&s_in)[2], float16v (&s_out)[2]) {
        const int jnn = (jn < nv) ? it_next() : nv;
        if (jnn < nv) issue_fp4(smem + ldslot * T::RING, jnn);
        if (head_ok) {
          // Issue order: every LDS operand read first (the next tile's K
          // operands, this tile's V operands), then this tile's softmax with
          // the next tile's QK MFMAs spread through it (in-order issue would
          // otherwise hold the VALU work behind back-to-back MFMAs), then
          // this tile's P.V MFMAs.  After the last tile the QK reads a stale
          // slot; its result is never used.
          int4v ka[2][D / 64], va[CB];
          int ks[2][D / 64], vs[CB];
          fp4_kops<D, HPW>(smem + nxt * T::RING, col, lh, ka, ks);
          fp4_vops<D, HPW>(smem + cur * T::RING, col, lh, va, vs);
          __builtin_amdgcn_sched_barrier(0);
          fp4_qk_mfma<D>(ka, ks, qf4, qs4, s_out);
          fp4_fixed_rest<CB>(s_in, va, vs, acc, M, l_part, overflow, c);
#pragma unroll
          for (int q = 0; q < 2 * (D / 64); q++) {
            __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);  // VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA (QK)
          }
        }
        wait_vmem();
        __syncthreads();
        jc = jn;
        jn = jnn;
      };
      while (pass == 0 && jc < nv) {
        step(0, 1, 2, sa, sb);
        if (jc >= nv) break;
        step(1, 2, 0, sb, sa);
        if (jc >= nv) break;
        step(2, 0, 1, sa, sb);
        if (jc >= nv) break;
        step(0, 1, 2, sb, sa);
        if (jc >= nv) break;
        step(1, 2, 0, sa, sb);
        if (jc >= nv) break;
        step(2, 0, 1, sb, sa);
      }
      // pass 1: the same walk, double-buffered, with the rescaling tile body
      int p1 = 0;
      while (pass == 1 && jc < nv) {
        if (jn < nv) issue_fp4(smem + (p1 ^ 1) * T::RING, jn);
        if (head_ok) tile_fp4<D, HPW, false>(smem + p1 * T::RING, qf4, qs4, acc, M, l_part, c, col, lh, qpos);
        wait_vmem();
        __syncthreads();
        p1 ^= 1;
        jc = jn;
        jn = (jn < nv) ? it_next() : nv;
      }
    }
    if (pass == 0 && __syncthreads_or(overflow ? 1 : 0)) continue;

    // ---- epilogue: O = acc / l, lse = (M + log2 l) ln 2
    if (!head_ok) return;
    const float l = l_part + other_half(l_part);
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
    return;
  }
}

template <int D, int HPW>
static hipError_t launch_one(const AttnArgs &a, hipStream_t st) {
  using T = Tile<D, HPW>;
  const int group = a.Hq / a.Hkv;
  const int chunks = (group + HPW - 1) / HPW;
  const size_t lds = (size_t)T::LDS;
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
