// Step 3 of the ThriftAttention path ("ThriftAttention: Selective Mixed
// Precision for Long-Context FP4 Attention", abstract): the selected
// query-key blocks are computed in FP16, the remaining ones in block-scaled
// 4-bit, and both paths are merged by one online softmax into one output.
//
// Work decomposition (gfx950, wave64): three kernels on one stream.
//   * attn_f16_kernel: one workgroup of 4 waves per (batch, query head,
//     query block i) walks the FP16 list of that row block (block 0 and the
//     diagonal block are always on it).  Each wave owns 32 query rows and
//     one 32-key half of every 64-key tile, with its own online softmax; the
//     two key halves are merged through LDS at the end and the partial state
//     (unnormalised O^T, M, the lane's row-sum part) goes to the workspace.
//   * attn_fwd_kernel: one workgroup per (batch, HPW query heads of one GQA
//     group, query block i); HPW = 2 over the pairs of a group's heads and 1
//     for the last head of an odd group.  It starts from those partial
//     states and walks, in
//     ascending order, every block that is on the FP4 list of at least one
//     of its heads, staging the block's MXFP4 K/V once for all of them.  A
//     wave owns 32 query rows of one head and computes the blocks on its own
//     head's FP4 list; the others are skipped.  It normalises and stores the
//     rows, unless the overflow rule below flags the workgroup.
//   * attn_redo_kernel: a small grid that reads every work item's flag and
//     recomputes the flagged ones from scratch with the general walk (every
//     block in ascending order, FP16 or FP4 per head, M raised by either kind).
// Every tile is S^T = K Q^T with 32x32 MFMAs (FP16: v_mfma_f32_32x32x16_f16;
// FP4: v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0 scales), then
// O^T += V^T P^T.
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
// re-quantization of P (a per-group power-of-two scale) unchanged.  FP16
// tiles (block 0 and the diagonal are always among them) raise M when their
// max exceeds it by more than kLazy (fp16 P stays below 2^kLazy).  FP4 tiles
// take p = 2^(x - M) against the M left by the FP16 tiles without raising
// it; their group scales absorb any p above 1.  If some p exceeds kMaxP, or
// the result is not finite, the work item is redone with the general walk,
// whose FP4 tiles raise M as well.
#include "thrift_internal.h"

namespace thrift {

constexpr float kLazy = 8.0f;
// Largest p an FP4 tile may take against the running max without raising
// it: P's E8M0 scale byte stays at most 127 + 100 - 2, the row sum below
// 2^(100 + 19); the accumulator is checked for overflow at the end.
constexpr float kMaxP = 0x1p100f;

template <int D, int HPW>
struct Tile {
  // FP4 tile, kept as two halves that are loaded and consumed at different
  // steps: a K slot (K codes | K scale bytes) and a V slot (V codes | V
  // scale bytes); the code regions are whole 1 KB groups.
  static constexpr int K4 = 64 * D / 2, K4S = 64 * D / 32, V4 = D * 32, V4S = D * 2;
  static constexpr int KSLOT = K4 + K4S, VSLOT = V4 + V4S;
  static constexpr int oK4 = 0, oK4S = K4;  // inside a K slot
  static constexpr int oV4 = 0, oV4S = V4;  // inside a V slot
  static constexpr int G4K = K4 / 1024, G4 = (K4 + V4) / 1024;  // 64-chunk groups of K codes, of K+V codes
  // FP16 tile: K rows | channel-major V
  static constexpr int K16 = 64 * D * 2, V16 = D * 64 * 2;
  static constexpr int FP16_BYTES = K16 + V16;
  static constexpr int oK16 = 0, oV16 = K16;
  static constexpr int G16 = FP16_BYTES / 1024;  // 64-chunk groups of an FP16 tile
  // Two slots of each kind (redo walk): the FP16 tile, K half and V half of
  // the block at walk position m sit in slot m % 2.
  static constexpr int oSLOT16 = 0, oKSLOT = 2 * FP16_BYTES, oVSLOT = oKSLOT + 2 * KSLOT;
  // then the workgroup's Q16 rows ([HPW*64][D] halves, 16-byte chunks
  // XOR-swizzled by row) and the FP16-list bitmasks
  static constexpr int oQ16 = oVSLOT + 2 * VSLOT;
  static constexpr int Q16_BYTES = HPW * 64 * D * 2;
  static constexpr int oMASK = oQ16 + Q16_BYTES;
  static constexpr int oIMASK = oMASK + HPW * (kMaxBlocks / 32) * 4;  // FP16 on every head
  static constexpr int LDS = oIMASK + (kMaxBlocks / 32) * 4;             // redo kernel
  // The FP4 kernel needs only the FP4 slots and the masks.
  static constexpr int f4KSLOT = 0, f4VSLOT = 2 * KSLOT, f4MASK = f4VSLOT + 2 * VSLOT;
  static constexpr int f4IMASK = f4MASK + HPW * (kMaxBlocks / 32) * 4;
  static constexpr int F4_LDS = f4IMASK + (kMaxBlocks / 32) * 4;
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
// K16 rows (D/8 chunks) are read in two patterns: the FP16 kernel's half
// tiles (16 lanes vary key bits 0-3) and the redo walk's permuted full tiles
// (16 lanes vary key bits 0, 1, 2 and 5).  Taking bit 3 ^ bit 5 into the map
// makes it one-to-one on both sets of bits at D = 128.
template <int D>
__device__ __forceinline__ int swz_k16(int key) {
  const int b35 = ((key >> 3) ^ (key >> 5)) & 1;
  if (D == 128) return (key & 3) | (b35 << 2) | (((key >> 2) & 1) << 3);
  return ((key >> 1) & 1) | (((key >> 2) & 1) << 1) | (b35 << 2);
}
__device__ __forceinline__ int swz_v16(int ch) { return (ch ^ (ch >> 3)) & 7; }       // V16 rows: 8 chunks
__device__ __forceinline__ int swz_v4(int ch) { return ((ch >> 2) ^ (ch >> 3)) & 1; }  // V4 rows: 2 chunks

// Key (row of the 64-key tile) that A-operand row rho of MFMA block blk
// reads, so that the result lands in the lane layout described above.
__device__ __forceinline__ int permuted_key(int rho, int blk) {
  return 32 * ((rho >> 2) & 1) + 16 * blk + 4 * (rho >> 3) + (rho & 3);
}

// Buffer resource over a byte array: base p, no stride, no range clamp
// (every offset the kernels form is inside the array).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, -1, 0x00020000);
}

// 16 bytes per lane from buffer offset voff + soff (soff wave-uniform)
// straight into LDS at byte address lds_wave_base + 16 * lane
// (lds_wave_base wave-uniform).  The LDS address is a plain 32-bit integer,
// so forming it needs no generic-to-LDS pointer conversion.
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff,
                                              uint32_t lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(size_t)lds_wave_base, 16,
                                           voff, soff, 0, 0);
}

// s_waitcnt immediate for vmcnt(n) alone (0 <= n < 64): the counter's low
// four bits sit in bits 3:0, its high two in bits 15:14; expcnt (6:4) and
// lgkmcnt (11:8) at their no-wait maxima.
constexpr int vmcnt_imm(const int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
static_assert(vmcnt_imm(0) == 0x0F70 && vmcnt_imm(16) == 0x4F70, "vmcnt encoding");

// Workgroup barrier after s_waitcnt vmcnt(n) lgkmcnt(0) (n < 64, a constant):
// this wave's LDS accesses are done and at most its n newest vector-memory
// loads are outstanding (direct-to-LDS copies that later steps wait for).
// Unlike __syncthreads() it does not drain every outstanding load; the empty
// asm statements keep the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void barrier_vmcnt() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N) & ~0x0F00);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Raise the integer running max M (log2 units) to ceil(row max * c) when it
// exceeds M by more than kLazy (or M is still -inf), rescaling acc and the
// row sum by the exact power of two.  lane_max: this lane's largest raw
// score (the row's other 32 keys sit in lane l ^ 32).
template <int CB>
__device__ __forceinline__ void raise_max(const float lane_max, float16v (&acc)[CB], float &M, float &l_part,
                                          const float c) {
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
}

// Online-softmax step on one 32-query x 64-key score tile held as s[2]
// (this lane: query col, keys 32*lh + 0..31).  Applies the causal mask on
// the diagonal tile, raises the integer running max when needed (rescaling
// acc and the row sum by an exact power of two), replaces s by
// p = 2^(s*c - M) and adds the lane's p to l_part.  Returns the lane's
// largest raw score (-inf if all masked).
// LS picks what the row sum adds: 0 the fp32 p, 1 fp16(p) (p is also left
// rounded to fp16 in s), 2 nothing (the caller adds the dequantized FP4 P).
template <int CB, bool MASK, int LS = 0>
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
  raise_max<CB>(lane_max, acc, M, l_part, c);
  const float negM = -M;
  float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s[0][r] = __builtin_amdgcn_exp2f(fmaf(s[0][r], c, negM));
    s[1][r] = __builtin_amdgcn_exp2f(fmaf(s[1][r], c, negM));
    if (LS == 1) {
      s[0][r] = (float)(_Float16)s[0][r];
      s[1][r] = (float)(_Float16)s[1][r];
    }
    l0 += s[0][r];
    l1 += s[1][r];
  }
  if (LS != 2) l_part += l0 + l1;
  return lane_max;
}

// Sum of the 32 E2M1 values packed in pw (this lane's P codes), times the
// group scale 2^(psb - 127): the lane's dequantized P.  The code sums are
// exact in fp32 (at most 32 * 6, multiples of 1/2).
__device__ __forceinline__ float fp4_code_sum(const uint32_t (&pw)[4], const int psb) {
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[w], 1.0f, 0);
    const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[w], 1.0f, 1);
    const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[w], 1.0f, 2);
    const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[w], 1.0f, 3);
    t += ((f0[0] + f0[1]) + (f1[0] + f1[1])) + ((f2[0] + f2[1]) + (f3[0] + f3[1]));
  }
  return ldexpf(t, psb - 127);
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

// LDS byte address (32-bit) of a pointer into the dynamic shared array, and
// reads at such an address: a register plus a constant offset folds into
// one ds_read.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
__device__ __forceinline__ int4v lds_read16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) int4v *)(size_t)addr;
}
__device__ __forceinline__ int lds_read8(uint32_t addr) {
  return *(const __attribute__((address_space(3))) uint8_t *)(size_t)addr;
}

// Per-lane LDS addresses of the FP4 MFMA operand reads in K slot 0 and V
// slot 0 (slot s adds s * KSLOT or s * VSLOT), so each read in the walk is
// one of eight registers plus a constant.
template <int D, int HPW>
struct Fp4Offsets {
  uint32_t k[2][D / 64];  // K codes of block blk, k-step kk
  uint32_t ks[2];         // K scale bytes of block blk (+ 2 kk)
  uint32_t v;             // V codes of channel block 0 (+ 1024 cb)
  uint32_t vs;            // V scale bytes of channel block 0 (+ 64 cb)
  __device__ __forceinline__ Fp4Offsets(const uint8_t *kslot0, const uint8_t *vslot0, const int col, const int lh) {
    using T = Tile<D, HPW>;
    const uint32_t kb = lds_addr(kslot0), vb = lds_addr(vslot0);
#pragma unroll
    for (int blk = 0; blk < 2; blk++) {
      const int key = permuted_key(col, blk);
#pragma unroll
      for (int kk = 0; kk < D / 64; kk++)
        k[blk][kk] = kb + T::oK4 + key * (D / 2) + 16 * ((2 * kk + lh) ^ swz_k4<D>(key));
      ks[blk] = kb + T::oK4S + key * (D / 32) + lh;
    }
    // swz_v4 of channel 32 cb + col depends on col only
    v = vb + T::oV4 + col * 32 + 16 * (lh ^ swz_v4(col));
    vs = vb + T::oV4S + col * 2 + lh;
    // opaque to the compiler, so that the walk keeps these addresses in
    // registers instead of re-deriving them with adds at every step
#pragma unroll
    for (int blk = 0; blk < 2; blk++) {
#pragma unroll
      for (int kk = 0; kk < D / 64; kk++) asm volatile("" : "+v"(k[blk][kk]));
      asm volatile("" : "+v"(ks[blk]));
    }
    asm volatile("" : "+v"(v));
    asm volatile("" : "+v"(vs));
  }
};

template <int D, int HPW>
__device__ __forceinline__ void fp4_kops_at(const int slot_off, const Fp4Offsets<D, HPW> &fo,
                                            int4v (&ka)[2][D / 64], int (&ks)[2][D / 64]) {
#pragma unroll
  for (int blk = 0; blk < 2; blk++)
#pragma unroll
    for (int kk = 0; kk < D / 64; kk++) {
      ka[blk][kk] = lds_read16(fo.k[blk][kk] + slot_off);
      ks[blk][kk] = lds_read8(fo.ks[blk] + slot_off + 2 * kk);
    }
}

template <int D, int HPW>
__device__ __forceinline__ void fp4_vops_at(const int slot_off, const Fp4Offsets<D, HPW> &fo, int4v (&va)[D / 32],
                                            int (&vs)[D / 32]) {
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) {
    va[cb] = lds_read16(fo.v + slot_off + 1024 * cb);
    vs[cb] = lds_read8(fo.vs + slot_off + 64 * cb);
  }
}

// FP4 tile, first half: S^T (masked on the diagonal) and the V operands
// (read here so their LDS latency hides under the softmax).
template <int D, int HPW, bool MASK>
__device__ __forceinline__ void fp4_scores(const uint8_t *kst, const uint8_t *vst, const int4v (&qf4)[D / 64], const int (&qs4)[D / 64],
                                           const int col, const int lh, const int qpos, float16v (&s)[2],
                                           int4v (&va)[D / 32], int (&vs)[D / 32]) {
  fp4_qk<D, HPW>(kst, qf4, qs4, col, lh, s);
  fp4_vops<D, HPW>(vst, col, lh, va, vs);
  if (MASK) {
#pragma unroll
    for (int blk = 0; blk < 2; blk++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (32 * lh + 16 * blk + r > qpos) s[blk][r] = -INFINITY;
  }
}

// The lane's 32 values of s (one aligned 32-key group), divided by div and
// rounded to E2M1, packed: byte b of word w holds keys 16(w/2) + 8(w%2) +
// 2b, +1 (low nibble first).
__device__ __forceinline__ void fp4_pack(const float16v (&s)[2], const float div, uint32_t (&pw)[4]) {
#pragma unroll
  for (int w = 0; w < 4; w++) {
    const int blk = w >> 1, r0 = 8 * (w & 1);
    // the four converts replace all four bytes; starting from s's own bits
    // leaves the register allocator nothing to initialise
    pw[w] = __float_as_uint(s[blk][r0]);
    THRIFT_CVT_FP4(pw[w], s[blk][r0 + 0], s[blk][r0 + 1], div, 0);
    THRIFT_CVT_FP4(pw[w], s[blk][r0 + 2], s[blk][r0 + 3], div, 1);
    THRIFT_CVT_FP4(pw[w], s[blk][r0 + 4], s[blk][r0 + 5], div, 2);
    THRIFT_CVT_FP4(pw[w], s[blk][r0 + 6], s[blk][r0 + 7], div, 3);
  }
}

// Exp-free codes of the lane's 32 raw scores s (the other row-sum reading's
// cheap FP4 path): the group exponent is the MX rule applied to the largest
// p = 2^(x_max - M) without forming it, e = floor(x_max - M) - 2 (clamped to
// [-127, 127]; -127 for an all-masked group), and each key's code is the
// E2M1 rounding of 2^floor(y) (1 + frac y), y = x - M - e.  That float is
// the bit pattern (y + 127) 2^23, so one fma (s c 2^23 + (127 - M - e) 2^23)
// and one saturating conversion to an integer give it; y <= -127 (and a
// masked -inf) saturate to 0.  Returns the scale byte e + 127; `big` is set
// when e exceeds the fixed-max walk's limit (p above 2^100).
__device__ __forceinline__ int fp4_log_codes(float16v (&s)[2], const float M, const float c, uint32_t (&pw)[4],
                                             bool &big) {
  const float xm = lane_max32(s) * c;
  int e = -127;
  if (xm != -INFINITY) e = min(max((int)floorf(xm - M) - 2, -127), 127);
  big = e > 98;
  const float c23 = c * 8388608.0f, k23 = (127.0f - M - (float)e) * 8388608.0f;
#pragma unroll
  for (int blk = 0; blk < 2; blk++)
#pragma unroll
    for (int r = 0; r < 16; r++) s[blk][r] = __uint_as_float((uint32_t)fmaf(s[blk][r], c23, k23));
  fp4_pack(s, 1.0f, pw);
  return e + 127;
}

// O^T += V^T P^T for the packed codes pw with scale byte psb.  WS 1: also adds
// the lane's dequantized P to *l_add (VALU); WS 2: also accumulates the
// dequantized P of every key into lacc with one more scaled MFMA against
// E2M1 ones (every row of lacc then holds the row's sum).
template <int CB, int WS = 0>
__device__ __forceinline__ void fp4_pv_codes(const uint32_t (&pw)[4], const int psb, const int4v (&va)[CB],
                                             const int (&vs)[CB], float16v (&acc)[CB], float *l_add = nullptr,
                                             float16v *lacc = nullptr) {
  int8v pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], 0, 0, 0, 0};
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    int8v a8 = {va[cb][0], va[cb][1], va[cb][2], va[cb][3], 0, 0, 0, 0};
    acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, pb, acc[cb], 4, 4, 0, vs[cb], 0, psb);
  }
  if (WS == 1) *l_add += fp4_code_sum(pw, psb);
  if (WS == 2) {
    // E2M1 code 2 (1.0) in every nibble, scale byte 127 (2^0)
    const int8v ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
    *lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, *lacc, 4, 4, 0, 127, 0, psb);
  }
}

// FP4 tile, second half: p (this lane's 32 values, one aligned 32-key group,
// relative to the max the exponent used, amax their largest) re-quantized to
// MXFP4, and O^T += V^T P^T (WS as fp4_pv_codes).
template <int CB, int WS = 0>
__device__ __forceinline__ void fp4_pv(const float16v (&s)[2], const float amax, const int4v (&va)[CB],
                                       const int (&vs)[CB], float16v (&acc)[CB], float *l_add = nullptr,
                                       float16v *lacc = nullptr) {
  const int psb = mx_scale_byte(amax);
  uint32_t pw[4];
  fp4_pack(s, mx_scale_divisor(psb), pw);
  fp4_pv_codes<CB, WS>(pw, psb, va, vs, acc, l_add, lacc);
}

// One FP4 tile (general walk): the running max may rise, rescaling acc.
// R: the row-sum reading (0 the unquantized p, 1 the weights P.V uses, 2 as
// 1 with exp-free P codes).
template <int D, int HPW, bool MASK, int R = 0>
__device__ __forceinline__ void tile_fp4(const uint8_t *kst, const uint8_t *vst, const int4v (&qf4)[D / 64], const int (&qs4)[D / 64],
                                         float16v (&acc)[D / 32], float &M, float &l_part, const float c,
                                         const int col, const int lh, const int qpos) {
  constexpr int CB = D / 32;
  float16v s[2];
  int4v va[CB];
  int vs[CB];
  fp4_scores<D, HPW, MASK>(kst, vst, qf4, qs4, col, lh, qpos, s, va, vs);
  if (R == 2) {
    raise_max<CB>(lane_max32(s), acc, M, l_part, c);
    uint32_t pw[4];
    bool big;
    const int psb = fp4_log_codes(s, M, c, pw, big);
    fp4_pv_codes<CB, 1>(pw, psb, va, vs, acc, &l_part);
  } else {
    const float lane_max = softmax_step<CB, false, R ? 2 : 0>(s, acc, M, l_part, c, lh, qpos);
    fp4_pv<CB, R ? 1 : 0>(s, __builtin_amdgcn_exp2f(fmaf(lane_max, c, -M)), va, vs, acc, &l_part);
  }
}

// Softmax and P.V of one FP4 tile whose scores s are already computed,
// against the running max M as it stands: p = 2^(s*c - M) is taken
// directly, so no step of the exponentials waits on this tile's max, and the
// accumulator is not rescaled.  p is summed into l_part unquantized; P's
// group scale comes from the largest p of the lane's 32-key group (the MXFP4
// rule's amax, taken after the exponentials).  A group with amax above kMaxP
// (or not finite) sets `overflow`.
template <int CB, int R = 0>
__device__ __forceinline__ void fp4_fixed_rest(float16v (&s)[2], const int4v (&va)[CB], const int (&vs)[CB],
                                               float16v (&acc)[CB], const float M, float &l_part, bool &overflow,
                                               const float c, float16v *lacc = nullptr) {
  if (R == 2) {  // exp-free codes; the row sum from the ones-MFMA
    uint32_t pw[4];
    bool big;
    const int psb = fp4_log_codes(s, M, c, pw, big);
    overflow = overflow || big;
    fp4_pv_codes<CB, 2>(pw, psb, va, vs, acc, nullptr, lacc);
    return;
  }
  constexpr bool W = R != 0;
  const float negM = -M;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s[0][r] = __builtin_amdgcn_exp2f(fmaf(s[0][r], c, negM));
    s[1][r] = __builtin_amdgcn_exp2f(fmaf(s[1][r], c, negM));
  }
  if (!W) {
    float l0 = s[0][0], l1 = s[1][0];
#pragma unroll
    for (int r = 1; r < 16; r++) {
      l0 += s[0][r];
      l1 += s[1][r];
    }
    l_part += l0 + l1;
  }
  const float amax = lane_max32(s);
  overflow = overflow || !(amax <= kMaxP);
  fp4_pv<CB, W ? 2 : 0>(s, amax, va, vs, acc, nullptr, lacc);
}

// True if x is an infinity or a NaN (exponent field all ones); integer test,
// so it holds whatever the compiler assumes about NaNs.
__device__ __forceinline__ bool not_finite(float x) { return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u; }

// One FP16 tile for one wave: S^T from FP16 K and Q, P rounded to fp16,
// O^T += V^T P^T with FP16 V.  st16 is the tile's FP16 region (K rows, then
// channel-major V); qrow16 points at this lane's Q16 row in LDS.
template <int D, int HPW, bool MASK, int R = 0>
__device__ __forceinline__ void tile_fp16(const uint8_t *st16, const uint8_t *qrow16, float16v (&acc)[D / 32],
                                          float &M, float &l_part, const float c, const int col_in, const int lh,
                                          const int qpos) {
  using T = Tile<D, HPW>;
  constexpr int KS = D / 16, CB = D / 32, CPR = D / 8;  // k-steps, channel blocks, 16-byte chunks per row
  // The per-lane operand addresses below are recomputed on every call: an
  // empty asm makes the lane index opaque here, so they are not hoisted out
  // of the walk loop (which would hold dozens of address registers across
  // the hot FP4 steps).
  int col_v = col_in;
  asm volatile("" : "+v"(col_v));
  const int col = col_v;
  float16v s[2];
#pragma unroll
  for (int blk = 0; blk < 2; blk++)
#pragma unroll
    for (int r = 0; r < 16; r++) s[blk][r] = 0.0f;
  const int key0 = permuted_key(col, 0), key1 = permuted_key(col, 1);
  const uint8_t *k0 = st16 + T::oK16 + key0 * (2 * D);
  const uint8_t *k1 = st16 + T::oK16 + key1 * (2 * D);
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
  softmax_step<CB, MASK, R ? 1 : 0>(s, acc, M, l_part, c, lh, qpos);
  // P in fp16; MFMA u consumes keys 32*lh + 8u + 0..7 of this lane
  half8 pb[4];
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int t = 0; t < 8; t++) pb[u][t] = (_Float16)s[u >> 1][8 * (u & 1) + t];
  const uint8_t *vt = st16 + T::oV16;
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

// Work item of one GQA workgroup: query block i of up to HPW heads of GQA
// group g in batch b (longest causal rows first).  The launch covers heads
// [a.hbase, a.hbase + a.hspan) of each group in chunks of hpw; this item
// holds group heads h0 .. h0 + nh - 1 (nh < hpw only in a last, partial
// chunk).
struct WorkItem {
  int i, b, g, h0, nh, nb, group, nv, nw;
  // item: the work item's index in its launch (the FP4 kernel's workgroup)
  __device__ __forceinline__ WorkItem(const AttnArgs &a, const int hpw, const int item) {
    nb = a.N / 64;
    group = a.Hq / a.Hkv;
    const int chunks = (a.hspan + hpw - 1) / hpw;
    const int per_i = a.B * a.Hkv * chunks;
    const int wi = item / per_i;
    int rem = item % per_i;
    i = a.causal ? nb - 1 - wi : wi;
    b = rem / (a.Hkv * chunks);
    rem %= a.Hkv * chunks;
    g = rem / chunks;
    const int chunk = rem % chunks;
    h0 = a.hbase + chunk * hpw;
    nh = min(hpw, a.hspan - chunk * hpw);
    nv = a.causal ? i + 1 : nb;
    nw = (nv + 31) / 32;
  }
};

// K/V tile loads: direct copies into LDS (buffer_load ... lds; lane L of a
// wave writes its 16 bytes at the wave-uniform LDS base + 16 L).  The array
// base of this KV head sits in a scalar buffer resource, the block offset
// j * (bytes per block) in a scalar register, and the per-lane offset inside
// the block (with the chunk swizzle of the region) in a VGPR.  The waves of a
// workgroup split a tile into whole 1 KB groups; the K and V scale bytes go
// to the last two waves (to the only wave if there is one).  The caller
// waits (vmcnt) before the barrier that publishes a tile.
template <int D, int NWAVES>
struct Loader {
  using T = Tile<D, 1>;
  static constexpr int NG4 = (T::G4 + NWAVES - 1) / NWAVES, NG16 = (T::G16 + NWAVES - 1) / NWAVES;
  static constexpr int KSW = NWAVES >= 2 ? NWAVES - 2 : 0, VSW = NWAVES - 1;  // scale-byte waves
  __amdgpu_buffer_rsrc_t rk4, rv4, rk4s, rv4s, rk16, rv16;
  int wave_u, lane;
  uint32_t goff4[NG4];
  __device__ __forceinline__ Loader(const AttnArgs &a, const int b, const int hkv, const int wave_u_, const int lane_)
      : wave_u(wave_u_), lane(lane_) {
    const int nb = a.N / 64;
    const int64_t kvh = (int64_t)b * a.Hkv + hkv;
    rk4 = make_rsrc(a.k4 + kvh * a.N * (D / 2));
    rv4 = make_rsrc(a.v4 + kvh * nb * (int64_t)(32 * D));
    rk4s = make_rsrc(a.k4s + kvh * a.N * (D / 32));
    rv4s = make_rsrc(a.v4s + kvh * nb * (int64_t)(2 * D));
    rk16 = make_rsrc((const uint8_t *)a.k16 + kvh * a.N * (2 * D));
    rv16 = make_rsrc((const uint8_t *)a.v16 + kvh * nb * (int64_t)(128 * D));
#pragma unroll
    for (int q = 0; q < NG4; q++) {
      const int t = wave_u + q * NWAVES;
      if (t < T::G4K) {
        const int off = 1024 * t + 16 * lane, key = off / (D / 2), pch = (off % (D / 2)) / 16;
        goff4[q] = key * (D / 2) + 16 * (pch ^ swz_k4<D>(key));
      } else {
        const int o = 1024 * (t - T::G4K) + 16 * lane, ch = o / 32, pch = (o % 32) / 16;
        goff4[q] = ch * 32 + 16 * (pch ^ swz_v4(ch));
      }
    }
  }
  // K half of block j's FP4 tile into the K slot at LDS address kst (codes
  // move by 32 D bytes per block, scale bytes by 2 D)
  __device__ __forceinline__ void k4(const uint32_t kst, const int j) const {
    __builtin_assume(wave_u >= 0 && wave_u < NWAVES);
#pragma unroll
    for (int q = 0; q < NG4; q++) {
      const int t = wave_u + q * NWAVES;
      if (t < T::G4K) buffer_to_lds(rk4, goff4[q], j * (32 * D), kst + 1024 * t);
    }
    if (wave_u == KSW && lane < T::K4S / 16) buffer_to_lds(rk4s, 16 * lane, j * (2 * D), kst + T::oK4S);
  }
  // V half of block j's FP4 tile into the V slot at LDS address vst
  __device__ __forceinline__ void v4(const uint32_t vst, const int j) const {
    __builtin_assume(wave_u >= 0 && wave_u < NWAVES);
#pragma unroll
    for (int q = 0; q < NG4; q++) {
      const int t = wave_u + q * NWAVES;
      if (t >= T::G4K && t < T::G4) buffer_to_lds(rv4, goff4[q], j * (32 * D), vst + 1024 * (t - T::G4K));
    }
    if (wave_u == VSW && lane < T::V4S / 16) buffer_to_lds(rv4s, 16 * lane, j * (2 * D), vst + T::oV4S);
  }
  // FP16 tile of block j into the FP16 slot at LDS address st16 (K16 and
  // V16 move by 128 D bytes per block); the per-lane offsets are formed here.
  __device__ __forceinline__ void fp16(const uint32_t st16, const int j) const {
    __builtin_assume(wave_u >= 0 && wave_u < NWAVES);
#pragma unroll
    for (int q = 0; q < NG16; q++) {
      const int t = wave_u + q * NWAVES;
      if (t < T::K16 / 1024) {
        const int off = 1024 * t + 16 * lane, key = off / (2 * D), pch = (off % (2 * D)) / 16;
        buffer_to_lds(rk16, key * (2 * D) + 16 * (pch ^ swz_k16<D>(key)), j * (128 * D), st16 + 1024 * t);
      } else if (t < T::G16) {
        const int o = 1024 * (t - T::K16 / 1024) + 16 * lane, ch = o / 128, pch = (o % 128) / 16;
        buffer_to_lds(rv16, ch * 128 + 16 * (pch ^ swz_v16(ch)), j * (128 * D), st16 + 1024 * t);
      }
    }
  }
};

// Heads of the workgroup with block j on their FP16 list (wave-uniform).
template <int HPW>
__device__ __forceinline__ uint32_t fp16_heads(const uint32_t *mask, const int j, const uint32_t head_bits) {
  uint32_t m = 0;
#pragma unroll
  for (int h = 0; h < HPW; h++) m |= ((mask[h * (kMaxBlocks / 32) + (j >> 5)] >> (j & 31)) & 1u) << h;
  return (uint32_t)__builtin_amdgcn_readfirstlane(m & head_bits);
}

// One wave's 32 query rows of Q16 into LDS at q16w (row-major, 16-byte
// chunks XOR-swizzled by row).
template <int D>
__device__ __forceinline__ void stage_q16(const AttnArgs &a, const int64_t qrow0, uint8_t *q16w, const int lane) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int it = 0; it < CPR / 2; it++) {  // 32 rows x CPR chunks over 64 lanes
    const int e = lane + 64 * it, row = e / CPR, ch = e % CPR;
    const int4v v = *(const int4v *)(a.q16 + (qrow0 + row) * D + 8 * ch);
    *(int4v *)(q16w + row * (2 * D) + 16 * (ch ^ (row & (CPR - 1)))) = v;
  }
}

// O = acc / l for this wave's 32 rows (lane: row col of the wave, channels
// 8(r/4) + 4(lane/32) + r%4 of each 32-channel block), lse = (M + log2 l) ln 2.
template <int D>
__device__ __forceinline__ void store_rows(const AttnArgs &a, const float16v (&acc)[D / 32], const float M,
                                           const float l_part, const int64_t qrow, const int lh) {
  constexpr int CB = D / 32;
  const float l = l_part + other_half(l_part);
  const float inv = 1.0f / l;
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const int ch = 32 * cb + 8 * q4 + 4 * lh;
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

// Partial state of one wave's 32 rows after its FP16 blocks, handed from the
// FP16 kernel to the FP4 kernel: per lane the D/2 accumulator values, the
// running max M and the lane's part of the row sum, stored field-major
// ([field][lane]) so both sides move whole 256-byte lines.
template <int D>
struct Partial {
  static constexpr int FIELDS = D / 2 + 2;
  static __device__ __forceinline__ float *at(float *ws, const int64_t wave_id) {
    return ws + wave_id * (int64_t)(FIELDS * 64);
  }
};

// ---------------------------------------------------------------------------
// FP16 kernel: one workgroup (four waves) per query block i of one head;
// walks the block's FP16 list (ascending, the diagonal last) and leaves the
// partial state in the workspace.  Split over keys: wave w owns query rows
// 32 (w & 1) + 0..31 and key half w >> 1 (keys 32 (w >> 1) + 0..31 of every
// tile) with an online softmax of its own; the two key halves of a row are
// merged at the end, so a tile needs no exchange between waves.
#ifndef THRIFT_F16_SLOTS
#define THRIFT_F16_SLOTS 2
#endif
template <int D>
struct Tile16 {
  static constexpr int FP16_BYTES = Tile<D, 1>::FP16_BYTES;
  static constexpr int SLOTS = THRIFT_F16_SLOTS;      // ring of FP16 tiles: SLOTS - 1 loads in flight
  static constexpr int LDS = SLOTS * FP16_BYTES;      // Q stays in registers
  static_assert(Partial<D>::FIELDS * 64 * 4 * 2 <= SLOTS * FP16_BYTES, "merge buffer fits in the slots");
};

// Online-softmax step on one 32-query x 32-key score tile s (this lane:
// query col, keys 16(r/8) + 8 lh + r%8 of the half): as softmax_step, for a
// tile in which every row has at least one valid key.
template <int CB, bool MASK, bool W>
__device__ __forceinline__ void softmax_half(float16v &s, float16v (&acc)[CB], float &M, float &l_part, const float c,
                                             const int key0, const int lh, const int qpos) {
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 16; r++)
      if (key0 + 16 * (r >> 3) + 8 * lh + (r & 7) > qpos) s[r] = -INFINITY;
  }
  float m0 = fmaxf(s[0], s[1]), m1 = fmaxf(s[8], s[9]);
#pragma unroll
  for (int r = 2; r < 8; r += 2) {
    m0 = fmaxf(fmaxf(m0, s[r]), s[r + 1]);
    m1 = fmaxf(fmaxf(m1, s[8 + r]), s[9 + r]);
  }
  const float lane_max = fmaxf(m0, m1);
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
  for (int r = 0; r < 8; r++) {
    s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, negM));
    s[8 + r] = __builtin_amdgcn_exp2f(fmaf(s[8 + r], c, negM));
    if (W) {  // the row sum adds the fp16 weights P.V uses
      s[r] = (float)(_Float16)s[r];
      s[8 + r] = (float)(_Float16)s[8 + r];
    }
    l0 += s[r];
    l1 += s[8 + r];
  }
  l_part += l0 + l1;
}

// One 32-key half (keys 32 kh + 0..31) of an FP16 tile for one wave: S^T from
// FP16 K (LDS; rows fed so that register r holds key 16(r/8) + 8 lh + r%8) and
// the lane's Q row (registers), P rounded to fp16, O^T += V^T P^T with FP16 V.
template <int D, bool MASK, bool W>
__device__ __forceinline__ void tile_fp16_half(const uint8_t *st16, const half8 (&qreg)[D / 16], const int kh,
                                               float16v (&acc)[D / 32], float &M, float &l_part, const float c,
                                               const int col, const int lh, const int qpos) {
  using T = Tile<D, 1>;
  constexpr int KS = D / 16, CB = D / 32;
  // A-operand row rho reads key 16(rho/16) + 8((rho/4)%2) + 4((rho/8)%2) + rho%4
  // of the half (bits 2 and 3 of rho swapped)
  const int key = 32 * kh + (col & 0x13) + ((col & 4) << 1) + ((col & 8) >> 1);
  const uint8_t *krow = st16 + T::oK16 + key * (2 * D);
  const int sw = swz_k16<D>(key);
  float16v s0, s1;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s0[r] = 0.0f;
    s1[r] = 0.0f;
  }
#pragma unroll
  for (int kk = 0; kk < KS; kk += 2) {
    half8 qb[2], ka[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int chunk = 2 * (kk + u) + lh;
      qb[u] = qreg[kk + u];
      ka[u] = __builtin_bit_cast(half8, *(const int4v *)(krow + 16 * (chunk ^ sw)));
    }
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[0], qb[0], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[1], qb[1], s1, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; r++) s0[r] += s1[r];
  softmax_half<CB, MASK, W>(s0, acc, M, l_part, c, 32 * kh, lh, qpos);
  // P in fp16: MFMA u consumes keys 16u + 8 lh + 0..7 (registers 8u + 0..7)
  half8 pb[2];
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int t = 0; t < 8; t++) pb[u][t] = (_Float16)s0[8 * u + t];
  const uint8_t *vt = st16 + T::oV16;
  // The P.V MFMAs issue at raised wave priority: a wave that reaches them
  // gets them into the matrix pipe ahead of the other wave's softmax work,
  // so it reaches the end-of-tile barrier (and the next tile's loads) sooner.
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    const int ch = 32 * cb + col;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const half8 vf =
          __builtin_bit_cast(half8, *(const int4v *)(vt + ch * 128 + 16 * ((4 * kh + 2 * u + lh) ^ swz_v16(ch))));
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pb[u], acc[cb], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int R>
__global__ __launch_bounds__(256) void attn_f16_kernel(AttnArgs a) {
  constexpr bool W = R != 0;  // the row sum adds fp16(p)
  using T = Tile<D, 1>;
  constexpr int CB = D / 32;
  constexpr int F = Partial<D>::FIELDS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nb = a.N / 64, group = a.Hq / a.Hkv;
  // KV-head-major order: the workgroups in flight at any time work on one
  // or two KV heads, whose FP16 K/V (128 N d bytes each) then stays in the
  // last-level cache while all their query heads and blocks read it.  Within
  // a KV head, longest causal rows first; with the round-robin dispatch over
  // the 8 XCDs, XCD x takes query blocks x, x+8, ... with all heads of the
  // group, so the blocks the heads share (the first and diagonal blocks, and
  // common picks) meet in one L2.
  const int kv = blockIdx.x / (nb * group), rem0 = blockIdx.x % (nb * group);
  // XCD (blockIdx % 8) takes every 8th query block with all heads of the group
  int wi, hh;
  if (nb % 8 == 0) {
    const int x = rem0 % 8, t = rem0 / 8;  // t-th item of XCD x
    hh = t % group;
    wi = 8 * (t / group) + x;
  } else {
    wi = rem0 / group;
    hh = rem0 % group;
  }
  const int b = kv / a.Hkv, hq = (kv % a.Hkv) * group + hh;
  const int bh = b * a.Hq + hq;
  const int i = a.causal ? nb - 1 - wi : wi;
  const int nv = a.causal ? i + 1 : nb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qhalf = wave_u & 1, kh = wave_u >> 1;
  const int col = lane & 31, lh = lane >> 5;
  const int qpos = 32 * qhalf + col;
  const int64_t qrow0 = ((int64_t)b * a.Hq + hq) * a.N + 64 * (int64_t)i + 32 * qhalf;

  const int64_t per = a.causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  const int64_t roff = a.causal ? (int64_t)i * (i + 1) / 2 : (int64_t)i * nb;
  // the list is read through the constant address space: scalar loads,
  // counted apart from the vector-memory loads of the tile ring
  typedef const __attribute__((address_space(4))) int32_t cint;
  cint *l16 = (cint *)(a.idx + (int64_t)bh * per + roff);
  const int cnt = min(max(((cint *)a.n16)[(int64_t)bh * nb + i], 0), nv);
  // This lane's Q row (query qrow0 + col) in registers, as the B operand of
  // the QK MFMAs: k-step kk takes channels 16 kk + 8 lh + 0..7.  Q is used
  // by every tile of the walk; reading it from LDS each time would be a
  // third of the kernel's LDS operand traffic.  A row block without FP16
  // blocks (cnt == 0, wave-uniform) loads nothing.
  half8 qreg[D / 16];
  if (cnt > 0) {
    const uint16_t *qr = a.q16 + (qrow0 + col) * D + 8 * lh;
#pragma unroll
    for (int kk = 0; kk < D / 16; kk++) qreg[kk] = __builtin_bit_cast(half8, *(const int4v *)(qr + 16 * kk));
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 16; kk++)
#pragma unroll
      for (int t = 0; t < 8; t++) qreg[kk][t] = (_Float16)0.0f;
  }
  // list entry e as a wave-uniform block index; an entry outside [0, nv)
  // (not produced by the selection) becomes -1 and is skipped: no load, no
  // tile, so every access stays inside this KV head's arrays
  auto entry = [&](int e) {
    const int j = l16[e];
    return ((unsigned)j < (unsigned)nv) ? j : -1;
  };
  const Loader<D, 4> ld(a, b, hq / group, wave_u, lane);

  float16v acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[cb][r] = 0.0f;
  float M = -INFINITY, l_part = 0.0f;
  // Ring of SLOTS FP16 tiles: list entry e in slot e % SLOTS; the loads of
  // entry e + SLOTS - 1 are issued while entry e is computed, and the wait
  // at the end of an entry keeps the newer entries' loads in flight.
  constexpr int RS = Tile16<D>::SLOTS;  // ring slots
  constexpr int LPT = Loader<D, 4>::NG16;  // load instructions per tile and wave
  int jq[RS];                                // blocks of entries e .. e + RS - 1 (-1: none or skipped)
#pragma unroll
  for (int q = 0; q < RS; q++) jq[q] = (q < cnt) ? entry(q) : -1;
#pragma unroll
  for (int q = 0; q < RS - 1; q++)
    if (jq[q] >= 0) ld.fp16(lds_addr(smem) + q * T::FP16_BYTES, jq[q]);
  wait_vmem();
  __syncthreads();
  // One step of the ring: finish entry e (its tile in slot e % RS) with the
  // loads of entry e + RS - 1 in flight.
  auto ring_step = [&](const int e, auto tile) {
    const int jl = jq[RS - 1];  // entry e + RS - 1
    if (jl >= 0) ld.fp16(lds_addr(smem) + ((e + RS - 1) % RS) * T::FP16_BYTES, jl);
    tile(smem + (e % RS) * T::FP16_BYTES, jq[0]);
    // entry e + 1 must have landed; entries e + 2 .. e + RS - 1 may stay in flight
    int inflight = 0;
#pragma unroll
    for (int q = 2; q < RS; q++) inflight += jq[q] >= 0 ? 1 : 0;
    if (RS < 3 || inflight == 0)
      barrier_vmcnt<0>();
    else if (RS < 4 || inflight == 1)
      barrier_vmcnt<LPT>();
    else
      barrier_vmcnt<2 * LPT>();
#pragma unroll
    for (int q = 0; q < RS - 1; q++) jq[q] = jq[q + 1];
    jq[RS - 1] = (e + RS < cnt) ? entry(e + RS) : -1;
  };
  // The list holds distinct blocks in ascending order, so entries before the
  // last are never the diagonal block (the last valid one): one unmasked
  // body in the loop; the last entry takes the masked body if it is the
  // diagonal.  jc is wave-uniform (a scalar branch); -1 marks a skipped entry.
  for (int e = 0; e + 1 < cnt; e++)
    ring_step(e, [&](const uint8_t *st16, int jc) {
      if (jc >= 0) tile_fp16_half<D, false, W>(st16, qreg, kh, acc, M, l_part, a.c, col, lh, qpos);
    });
  if (cnt > 0)
    ring_step(cnt - 1, [&](const uint8_t *st16, int jc) {
      if (jc < 0) return;
      if (a.causal && jc == i) {
        // the upper key half of the diagonal has no valid key for the lower rows
        if (!(kh == 1 && qhalf == 0)) tile_fp16_half<D, true, W>(st16, qreg, kh, acc, M, l_part, a.c, col, lh, qpos);
      } else {
        tile_fp16_half<D, false, W>(st16, qreg, kh, acc, M, l_part, a.c, col, lh, qpos);
      }
    });
  // Merge the two key halves of each row (lane by lane: the same lane of the
  // two waves holds the same query and channels) through the slot memory,
  // then the lower-half wave stores the row's partial state.
  float *xch = (float *)smem + (size_t)qhalf * F * 64;
  if (kh == 1) {
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) xch[(16 * cb + r) * 64 + lane] = acc[cb][r];
    xch[(D / 2) * 64 + lane] = M;
    xch[(D / 2 + 1) * 64 + lane] = l_part;
  }
  __syncthreads();
  if (kh == 0) {
    const float M1 = xch[(D / 2) * 64 + lane], l1 = xch[(D / 2 + 1) * 64 + lane];
    const float Mn = fmaxf(M, M1);
    // a half that saw no key has M = -inf and contributes nothing
    const float s0 = (M == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(M - Mn));
    const float s1 = (M1 == -INFINITY) ? 0.0f : ldexpf(1.0f, (int)(M1 - Mn));
    float *pw = Partial<D>::at(a.ws, ((int64_t)bh * nb + i) * 2 + qhalf);
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        pw[(16 * cb + r) * 64 + lane] = acc[cb][r] * s0 + xch[(16 * cb + r) * 64 + lane] * s1;
    pw[(D / 2) * 64 + lane] = Mn;
    pw[(D / 2 + 1) * 64 + lane] = l_part * s0 + l1 * s1;
  }
}

// FP16-list bitmask of each head of a GQA workgroup in LDS:
// mask[h][j/32] bit j%32 set when block j is on head h's FP16 list.  Ends
// with a barrier.
template <int HPW>
__device__ __forceinline__ void build_masks(const AttnArgs &a, const WorkItem &w, uint32_t *mask) {
  constexpr int NT = 128 * HPW;
  const int tid = threadIdx.x;
  for (int e = tid; e < HPW * w.nw; e += NT) mask[(e / w.nw) * (kMaxBlocks / 32) + e % w.nw] = 0;
  __syncthreads();
  const int64_t per = a.causal ? (int64_t)w.nb * (w.nb + 1) / 2 : (int64_t)w.nb * w.nb;
  const int64_t roff = a.causal ? (int64_t)w.i * (w.i + 1) / 2 : (int64_t)w.i * w.nb;
  for (int h = 0; h < HPW; h++) {
    if (h >= w.nh) break;
    const int hg = w.h0 + h;
    const int64_t bh = (int64_t)w.b * a.Hq + w.g * w.group + hg;
    // at most the row's n_valid entries (the FP16 kernel reads the same ones)
    const int cnt = min(max(a.n16[bh * w.nb + w.i], 0), w.nv);
    const int32_t *l16 = a.idx + bh * per + roff;
    for (int e = tid; e < cnt; e += NT) {
      const int j = l16[e];
      if ((unsigned)j < (unsigned)w.nv) atomicOr(&mask[h * (kMaxBlocks / 32) + (j >> 5)], 1u << (j & 31));
    }
  }
  __syncthreads();
}

// This launch's redo flags in the workspace (after the partial state),
// indexed by FP4 workgroup.
__device__ __forceinline__ int *redo_flags(const AttnArgs &a) {
  return (int *)(a.ws + (size_t)a.B * a.Hq * (a.N / 64) * 2 * 64 * (a.d / 2 + 2)) + a.fbase;
}

// ---------------------------------------------------------------------------
// Redo kernel: for the work items whose fixed-max FP4 walk flagged an
// overflow, the full walk over all blocks, FP16 and FP4, double-buffered
// (block j in slots j % 2), with tile bodies that raise M whenever a block
// needs it; then the rows are stored.  Same grid as the FP4 kernel; a
// workgroup whose item was not flagged returns at once.
// One flagged work item of the redo walk (smem: the workgroup's LDS).
template <int D, int HPW, int R>
__device__ __forceinline__ void redo_item(const AttnArgs &a, const int item, uint8_t *smem) {
  using T = Tile<D, HPW>;
  constexpr int KS4 = D / 64, CB = D / 32;
  const WorkItem w(a, HPW, item);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave_u >> 1, qhalf = wave_u & 1;
  const bool head_ok = hl < w.nh;
  const int hq = w.g * w.group + w.h0 + (head_ok ? hl : 0);
  const int col = lane & 31, lh = lane >> 5;
  const uint32_t head_bits = (1u << w.nh) - 1;
  uint32_t *mask = (uint32_t *)(smem + T::oMASK);
  build_masks<HPW>(a, w, mask);
  const int64_t qrow0 = ((int64_t)w.b * a.Hq + hq) * a.N + 64 * (int64_t)w.i + 32 * qhalf;
  const int64_t qrow = qrow0 + col;
  uint8_t *q16w = smem + T::oQ16 + (size_t)wave_u * 32 * D * 2;
  stage_q16<D>(a, qrow0, q16w, lane);
  const uint8_t *qrow16 = q16w + col * (2 * D);
  const int qpos = 32 * qhalf + col;
  int4v qf4[KS4];
  int qs4[KS4];
#pragma unroll
  for (int kk = 0; kk < KS4; kk++) {
    qf4[kk] = *(const int4v *)(a.q4 + qrow * (D / 2) + 32 * kk + 16 * lh);
    qs4[kk] = a.q4s[qrow * (D / 32) + 2 * kk + lh];
  }
  const Loader<D, 2 * HPW> ld(a, w.b, w.g, wave_u, lane);
  uint8_t *const slot16 = smem + T::oSLOT16, *const kslot = smem + T::oKSLOT, *const vslot = smem + T::oVSLOT;
  const float c = a.c;
  float16v acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[cb][r] = 0.0f;
  float M = -INFINITY, l_part = 0.0f;
  const int nv = w.nv;
  uint32_t hc = fp16_heads<HPW>(mask, 0, head_bits);
  const uint32_t slot16_a = lds_addr(slot16), kslot_a = lds_addr(kslot), vslot_a = lds_addr(vslot);
  if (hc != 0u) ld.fp16(slot16_a, 0);
  if (hc != head_bits) {
    ld.k4(kslot_a, 0);
    ld.v4(vslot_a, 0);
  }
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < nv; j++) {
    const int sl = j & 1, sn = sl ^ 1;
    const uint32_t hn = (j + 1 < nv) ? fp16_heads<HPW>(mask, j + 1, head_bits) : 0u;
    if (j + 1 < nv) {
      if (hn != 0u) ld.fp16(slot16_a + sn * T::FP16_BYTES, j + 1);
      if (hn != head_bits) {
        ld.k4(kslot_a + sn * T::KSLOT, j + 1);
        ld.v4(vslot_a + sn * T::VSLOT, j + 1);
      }
    }
    if (head_ok) {
      const bool fc = (hc >> hl) & 1u;
      const uint8_t *s16 = slot16 + sl * T::FP16_BYTES, *ks4 = kslot + sl * T::KSLOT, *vs4 = vslot + sl * T::VSLOT;
      if (a.causal && j == nv - 1) {
        if (fc)
          tile_fp16<D, HPW, true, R>(s16, qrow16, acc, M, l_part, c, col, lh, qpos);
        else
          tile_fp4<D, HPW, true, R>(ks4, vs4, qf4, qs4, acc, M, l_part, c, col, lh, qpos);
      } else {
        if (fc)
          tile_fp16<D, HPW, false, R>(s16, qrow16, acc, M, l_part, c, col, lh, qpos);
        else
          tile_fp4<D, HPW, false, R>(ks4, vs4, qf4, qs4, acc, M, l_part, c, col, lh, qpos);
      }
    }
    wait_vmem();
    __syncthreads();
    hc = hn;
  }
  if (head_ok) store_rows<D>(a, acc, M, l_part, qrow, lh);
}

// The redo walk over the FP4 launch's `items` work items: workgroup w takes
// the run of `per` items from w * per (per <= its thread count), reads their
// flags at once (one per thread) and, in the common case that none is set,
// exits after one barrier; otherwise it redoes the flagged ones in turn.  A
// small grid keeps the common case to a few microseconds.
template <int D, int HPW, int R>
__global__ __launch_bounds__(128 * HPW) void attn_redo_kernel(AttnArgs a, const int items, const int per) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int first = (int)blockIdx.x * per;
  const int n = min(per, items - first);
  const int f = ((int)threadIdx.x < n) ? redo_flags(a)[first + threadIdx.x] : 0;
  if (!__syncthreads_or(f)) return;
  for (int k = 0; k < n; k++) {
    if (redo_flags(a)[first + k] == 0) continue;  // the same value for every thread
    redo_item<D, HPW, R>(a, first + k, smem);
    __syncthreads();  // the next item rewrites the masks and tiles in LDS
  }
}

// ---------------------------------------------------------------------------
// FP4 kernel: one workgroup per query block i of HPW heads of a GQA group
// (a wave owns 32 rows of one head).  Each wave starts from the partial state
// its head's FP16 blocks left in the workspace and walks, ascending, every
// block below the diagonal that some head of the workgroup has on its FP4
// list, the next block's K/V tiles loading during each step.  The walk is the same for
// all waves (K/V tiles are shared in LDS); a head skips a block of its own
// FP16 list by adding neither p to l nor P.V to the accumulator.
template <int D, int HPW, int R>
__global__ __launch_bounds__(128 * HPW) void attn_fwd_kernel(AttnArgs a) {
  constexpr bool W = R != 0;  // the row sum adds the weights P.V uses
  using T = Tile<D, HPW>;
  constexpr int NT = 128 * HPW;                  // threads
  constexpr int KS4 = D / 64;                    // k-steps of the FP4 QK product
  constexpr int CB = D / 32;                     // 32-channel blocks of O^T

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t *mask = (uint32_t *)(smem + T::f4MASK);  // [HPW][kMaxBlocks/32] FP16-list bits
  uint32_t *imask = (uint32_t *)(smem + T::f4IMASK);  // blocks on every head's FP16 list

  const WorkItem w(a, HPW, (int)blockIdx.x);
  const int i = w.i, b = w.b, g = w.g, nb = w.nb, group = w.group, nv = w.nv, nw = w.nw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave_u >> 1, qhalf = wave_u & 1;
  const bool head_ok = hl < w.nh;
  const int hq = g * group + w.h0 + (head_ok ? hl : 0);
  const int col = lane & 31, lh = lane >> 5;

  const int64_t qrow = ((int64_t)b * a.Hq + hq) * a.N + 64 * (int64_t)i + 32 * qhalf + col;
  int4v qf4[KS4];
  int qs4[KS4];
#pragma unroll
  for (int kk = 0; kk < KS4; kk++) {
    qf4[kk] = *(const int4v *)(a.q4 + qrow * (D / 2) + 32 * kk + 16 * lh);
    qs4[kk] = a.q4s[qrow * (D / 32) + 2 * kk + lh];
  }
  // ---- FP16-list bitmask of each head of the workgroup
  build_masks<HPW>(a, w, mask);
  const uint32_t head_bits = (1u << w.nh) - 1;
  for (int e = tid; e < nw; e += NT) {
    uint32_t m = ~0u;
#pragma unroll
    for (int h = 0; h < HPW; h++)
      if ((head_bits >> h) & 1u) m &= mask[h * (kMaxBlocks / 32) + e];
    imask[e] = m;
  }
  // this wave's head's FP16 bits
  const uint32_t *own = mask + hl * (kMaxBlocks / 32);

  // ---- partial state of this wave's rows from the FP16 kernel
  float16v acc[CB];
  float M, l_part;
  {
    const int64_t bh = (int64_t)b * a.Hq + hq;
    const float *pw = Partial<D>::at(a.ws, (bh * nb + i) * 2 + qhalf);
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[cb][r] = pw[(16 * cb + r) * 64 + lane];
    M = pw[(D / 2) * 64 + lane];
    l_part = pw[(D / 2 + 1) * 64 + lane];
  }
  bool overflow = false;
  // row sums of the dequantized FP4 P of the fixed walk (weights row sum):
  // every row of this MFMA tile holds the lane's column sum
  float16v lacc;
#pragma unroll
  for (int r = 0; r < 16; r++) lacc[r] = 0.0f;
  __syncthreads();

  const Loader<D, 2 * HPW> ld(a, b, g, wave_u, lane);
  const float c = a.c;
  const int qpos = 32 * qhalf + col;  // query row inside the block
  uint8_t *const kslot = smem + T::f4KSLOT, *const vslot = smem + T::f4VSLOT;
  const uint32_t kslot_a = lds_addr(smem) + T::f4KSLOT, vslot_a = lds_addr(smem) + T::f4VSLOT;
  // The walk covers [0, jend); causal rows end at the diagonal block, whose
  // FP4 heads (if any) take the masked body after the walk.
  const int jend = a.causal ? nv - 1 : nv;

  // ---- the walk's blocks: not on every head's FP16 list, below jend; read
  // one 32-block word at a time, kept in a scalar register
  int it_w = 0;
  uint32_t it_bits = 0;  // unvisited blocks of word it_w
  uint32_t it_own = 0;   // this wave's head's FP16 bits of word it_w
  auto it_load = [&](int wd) {
    it_w = wd;
    uint32_t m = (wd < nw) ? ~(uint32_t)__builtin_amdgcn_readfirstlane(imask[wd]) : 0u;
    const int hi = jend - 32 * wd;  // blocks of this word below jend
    if (hi < 32) m &= hi > 0 ? ((1u << hi) - 1u) : 0u;
    it_bits = m;
    it_own = (wd < nw) ? (uint32_t)__builtin_amdgcn_readfirstlane(own[wd]) : 0u;
  };
  // Next block of the walk in ascending order (else nv), and whether this
  // wave's head has it on its FP4 list (so the flag is known steps ahead).
  uint32_t live_q = 0;  // FP4 flags of the blocks handed out, newest in bit 0
  auto it_next = [&]() -> int {
    while (it_bits == 0) {
      if (it_w + 1 >= nw) {
        live_q <<= 1;
        return nv;
      }
      it_load(it_w + 1);
    }
    const int b = __builtin_ctz(it_bits);
    it_bits &= it_bits - 1;
    live_q = (live_q << 1) | ((it_own >> b) & 1u ? 0u : 1u);
    return 32 * it_w + b;
  };
  it_load(0);
  int j0 = it_next();  // block of walk position m
  if (j0 < nv) {
    ld.k4(kslot_a, j0);
    ld.v4(vslot_a, j0);
  }
  wait_vmem();
  __syncthreads();
  if (j0 < nv) {
    float16v s0[2];
    fp4_qk<D, HPW>(kslot, qf4, qs4, col, lh, s0);
    // a row without FP16 blocks takes its M from this first tile
    const float lm = lane_max32(s0);
    const float mt = ceilf(fmaxf(lm, other_half(lm)) * c);
    M = (M == -INFINITY) ? mt : M;
  }
  const Fp4Offsets<D, HPW> fo(kslot, vslot, col, lh);
  // One FP4 block in slot k: QK, softmax against the fixed M, P.V.  The
  // next block's QK is not started early: that would keep a second score
  // tile live and cost the third wave per SIMD, which hides these latencies
  // better.
  auto block = [&](const int k) {
    float16v s[2];
    {
      int4v ka[2][D / 64];
      int ks[2][D / 64];
      fp4_kops_at<D, HPW>(k * T::KSLOT, fo, ka, ks);
      fp4_qk_mfma<D>(ka, ks, qf4, qs4, s);
    }
    int4v va[CB];
    int vs[CB];
    fp4_vops_at<D, HPW>(k * T::VSLOT, fo, va, vs);
    fp4_fixed_rest<CB, R>(s, va, vs, acc, M, l_part, overflow, c, &lacc);
  };
  // Step at walk position m (slot m % 2): loads the K and V of position m+1
  // into the other slot, then finishes position m if this wave's head has
  // it on its FP4 list (a block walked only for the other head is skipped).
  auto step = [&](const int k) {
    const int kn = k ^ 1;
    const int j1 = it_next();
    if (j1 < nv) {
      ld.k4(kslot_a + kn * T::KSLOT, j1);
      ld.v4(vslot_a + kn * T::VSLOT, j1);
    }
    if (head_ok && ((live_q >> 1) & 1u)) block(k);  // flag of j0, one behind j1's
    wait_vmem();
    __syncthreads();
    j0 = j1;
  };
  while (j0 < nv) {
    step(0);
    if (j0 >= nv) break;
    step(1);
  }
  // both lane halves hold the full column sum: one half adds it
  if (W && lh == 0) l_part += lacc[0];
  // the diagonal block (causal) for heads that have it on their FP4 list
  if (a.causal) {
    const uint32_t hd = fp16_heads<HPW>(mask, jend, head_bits);
    if (hd != head_bits) {
      ld.k4(kslot_a, jend);
      ld.v4(vslot_a, jend);
      wait_vmem();
      __syncthreads();
      if (head_ok && !((hd >> hl) & 1u))
        tile_fp4<D, HPW, true, R>(kslot, vslot, qf4, qs4, acc, M, l_part, c, col, lh, qpos);
    }
  }
  // An FP4 group above kMaxP, or an accumulator or row sum that left the
  // fp32 range, leaves the work item to the redo kernel (flag in the
  // workspace, written for every work item).
  bool bad = overflow || not_finite(l_part);
#pragma unroll
  for (int cb = 0; cb < CB; cb++)
#pragma unroll
    for (int r = 0; r < 16; r++) bad = bad || not_finite(acc[cb][r]);
  const int flagged = __syncthreads_or(bad ? 1 : 0);
  if (tid == 0) redo_flags(a)[blockIdx.x] = flagged;
  if (!flagged && head_ok) store_rows<D>(a, acc, M, l_part, qrow, lh);
}

// Redo launch over `items` FP4 work items with `threads` per workgroup:
// about kRedoGrid workgroups, each a run of at most `threads` items.
constexpr unsigned kRedoGrid = 2048;
struct RedoGrid {
  unsigned grid;
  int per;
  RedoGrid(const unsigned items, const unsigned threads) {
    unsigned g = items < kRedoGrid ? items : kRedoGrid;
    const unsigned need = (items + threads - 1) / threads;  // runs no longer than a workgroup
    g = g > need ? g : need;
    per = (int)((items + g - 1) / g);
    grid = (items + (unsigned)per - 1) / (unsigned)per;  // every workgroup has at least one item
  }
};

template <int D, int HPW, int R>
static hipError_t set_fp4_attrs() {
  using T = Tile<D, HPW>;
  hipError_t e = hipFuncSetAttribute((const void *)attn_fwd_kernel<D, HPW, R>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, T::F4_LDS);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void *)attn_redo_kernel<D, HPW, R>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             T::LDS);
}

// The FP16 kernel over every (b, query head, query block); then the FP4
// kernel over pairs of heads of each GQA group in two-head workgroups and,
// for an odd group, its last head in one-head workgroups (no wave of a
// two-head workgroup idles); then the redo kernels over the same grids.
// ev (nullable): four caller-created events recorded on st before the FP16
// kernel, between the kernels and after the redo kernels.
template <int D, int R>
static hipError_t launch_d(const AttnArgs &a, hipStream_t st, hipEvent_t const *ev) {
  const int group = a.Hq / a.Hkv;
  const int pairs = group / 2, single = group % 2;
  const unsigned nb = (unsigned)(a.N / 64);
  const unsigned per_head = nb * (unsigned)(a.B * a.Hkv);  // workgroups per head of a group
  AttnArgs a2 = a, a1 = a;
  a2.hbase = 0;
  a2.hspan = 2 * pairs;
  a2.fbase = 0;
  a1.hbase = 2 * pairs;
  a1.hspan = single;
  a1.fbase = (int)(per_head * (unsigned)pairs);
  const dim3 grid2(per_head * (unsigned)pairs), grid1(per_head);
  constexpr int R16 = R ? 1 : 0;  // FP16 tiles: readings 1 and 2 add fp16(p) alike
  hipError_t e = hipFuncSetAttribute((const void *)attn_f16_kernel<D, R16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Tile16<D>::LDS);
  if (e != hipSuccess) return e;
  if (pairs && (e = set_fp4_attrs<D, 2, R>()) != hipSuccess) return e;
  if (single && (e = set_fp4_attrs<D, 1, R>()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  hipLaunchKernelGGL((attn_f16_kernel<D, R16>), dim3(nb * (unsigned)(a.B * a.Hq)), dim3(256), Tile16<D>::LDS, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  if (pairs) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, 2, R>), grid2, dim3(256), (Tile<D, 2>::F4_LDS), st, a2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (single) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, 1, R>), grid1, dim3(128), (Tile<D, 1>::F4_LDS), st, a1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if (pairs) {
    const RedoGrid r2(grid2.x, 256);
    hipLaunchKernelGGL((attn_redo_kernel<D, 2, R>), dim3(r2.grid), dim3(256), (Tile<D, 2>::LDS), st, a2,
                       (int)grid2.x, r2.per);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (single) {
    const RedoGrid r1(grid1.x, 128);
    hipLaunchKernelGGL((attn_redo_kernel<D, 1, R>), dim3(r1.grid), dim3(128), (Tile<D, 1>::LDS), st, a1,
                       (int)grid1.x, r1.per);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev) e = hipEventRecord(ev[3], st);
  return e;
}

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t st, hipEvent_t const *ev) {
  if (a.d == 128) {
    if (a.rowsum == 2) return launch_d<128, 2>(a, st, ev);
    return a.rowsum ? launch_d<128, 1>(a, st, ev) : launch_d<128, 0>(a, st, ev);
  }
  if (a.rowsum == 2) return launch_d<64, 2>(a, st, ev);
  return a.rowsum ? launch_d<64, 1>(a, st, ev) : launch_d<64, 0>(a, st, ev);
}

size_t attn_workspace_bytes(const int B, const int Hq, const int N, const int d) {
  // partial states, then one redo flag per FP4 workgroup (at most B * Hq * N/64)
  return (size_t)B * Hq * (N / 64) * 2 * 64 * (size_t)(d / 2 + 2) * sizeof(float) +
         (size_t)B * Hq * (N / 64) * sizeof(int);
}

}  // namespace thrift
