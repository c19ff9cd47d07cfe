/*
 * thrift.h -- C ABI of the MI355X (gfx950) ThriftAttention prefill library.
 *
 * The method ("ThriftAttention: Selective Mixed Precision for Long-Context
 * FP4 Attention", abstract): a cheap heuristic first marks the few
 * query-key block pairs that matter most; those run at FP16 precision and
 * every other causally valid block in block-scaled 4-bit, and one online
 * softmax combines the two kinds of block into the result.  The
 * three calls below are the three steps of that path:
 *
 *   thrift_quantize   FP16 copies of Q/K/V and their MXFP4 codes
 *   thrift_select     the block heuristic: FP16 and FP4 traversal lists
 *   thrift_attn_fwd   fused mixed-precision attention with one online softmax
 *                     (thrift_attn_fwd_wsum: the same, normalised by the
 *                     quantized weights)
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned and allocated by the caller;
 *     the library allocates nothing, keeps no state between calls and never
 *     synchronizes.  All work is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream) and is asynchronous; calls are reentrant.  A call
 *     makes the stream's GPU current while it launches and the caller's
 *     device current again before it returns.
 *   - Every pointer must be 16-byte aligned.
 *   - Return value: THRIFT_OK (0) or a negative thrift_status.  Arguments are
 *     validated on the host before anything is enqueued, so an error return
 *     other than THRIFT_EHIP means nothing was launched.  THRIFT_EHIP reports
 *     a HIP launch error (hipGetLastError after the launch).
 *   - Shapes: B, Hq, Hkv, N > 0; Hq % Hkv == 0 (query head h reads KV head
 *     floor(h * Hkv / Hq)); d in {64, 128}; block == 64; N % 64 == 0;
 *     causal in {0, 1}; N / 64 <= 8192 and B * Hq * N / 64 < 2^24 (one
 *     workgroup per query block and head); otherwise THRIFT_EINVAL (bad
 *     values) or THRIFT_EUNSUPPORTED (valid but not built: other d, block,
 *     N % 64 != 0, beyond those sizes).
 *   - Inputs must be finite with |x| <= 65504; other values give undefined
 *     output but no out-of-bounds access.
 *   - nb = N / 64 blocks.  MXFP4 = OCP MX: E2M1 codes (sign bit 3, element
 *     2j of a group in the low nibble of byte j) with one E8M0 scale byte per
 *     32 elements; scale exponent = floor(log2 amax) - 2 (byte 0 for an
 *     all-zero group), elements rounded to nearest-even on the E2M1 grid and
 *     saturated to +-6.  One exception, inside thrift_attn_fwd only: a group
 *     of re-quantized P whose largest weight is below 2^-124 (scale byte 0)
 *     gets all-zero codes, where the rule would keep codes for its weights
 *     from 2^-129 up.  Such a group's weights are below 2^-119 of the row's
 *     largest, far under the output tolerance; Q, K and V groups (fp16 or
 *     bf16 values, |x| >= 2^-24 when non-zero) never reach byte 0 unless
 *     they are all zero.
 */
#ifndef THRIFT_H
#define THRIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  THRIFT_OK = 0,
  THRIFT_EINVAL = -1,      /* null/misaligned pointer, bad value */
  THRIFT_EUNSUPPORTED = -2,/* a shape this build does not handle */
  THRIFT_EWORKSPACE = -3,  /* workspace missing or too small */
  THRIFT_EHIP = -4         /* HIP launch error */
} thrift_status;

typedef enum { THRIFT_F16 = 0, THRIFT_BF16 = 1, THRIFT_F32 = 2 } thrift_dtype;

/* Block scores for the selection heuristic (thrift_select uses the pooled
 * mean; the others are the variants of thrift_select_ex). */
typedef enum {
  THRIFT_SCORE_POOLED_MEAN = 0,   /* pooled Q mean . pooled K mean */
  THRIFT_SCORE_MAX_POOLED = 1,    /* max over the key block's rows r of (pooled Q mean . k_r) */
  THRIFT_SCORE_NORM_WEIGHTED = 2, /* means with each row weighted by its L2 norm */
  THRIFT_SCORE_BLOCK_MAX = 3      /* largest exact q . k of the block pair (needs all of Q K^T) */
} thrift_score;

/* Problem statement: batch, query heads, KV heads, tokens, head dim, block
 * size (must be 64), causal mask flag. */
typedef struct {
  int32_t B, Hq, Hkv, N, d, block, causal;
} thrift_shape;

/*
 * Step 1 -- quantize (the block-scaled 4-bit operands of the FP4 path and the
 * FP16 operands of the FP16 path; the abstract names block-scaled 4-bit
 * quantisation as the prior art it builds on).
 *
 * in_dtype: THRIFT_F16 or THRIFT_BF16 for q, k, v.
 * Inputs (row-major): q [B,Hq,N,d], k and v [B,Hkv,N,d].
 * Outputs (all written completely):
 *   q16 [B,Hq,N,d], k16 [B,Hkv,N,d]   fp16, nearest-even rounding of the input
 *   v16 [B,Hkv,nb,d,64]               fp16, per 64-token block channel-major
 *                                     (element (t, c) at [t/64][c][t%64])
 *   q4 [B,Hq,N,d/2], q4s [B,Hq,N,d/32]     MXFP4 of q16, groups of 32 channels
 *   k4 [B,Hkv,N,d/2], k4s [B,Hkv,N,d/32]   MXFP4 of k16, groups of 32 channels
 *   v4 [B,Hkv,nb,d,32], v4s [B,Hkv,nb,d,2] MXFP4 of v16, groups of 32 tokens of
 *                                     one channel (token 64n + 32g + e is
 *                                     element e of group g of block n)
 * Errors: THRIFT_EINVAL for a null or misaligned pointer or a bad dtype.
 */
int thrift_quantize(const thrift_shape *s, int in_dtype, const void *q, const void *k, const void *v,
                    void *q16, void *k16, void *v16, void *q4, void *q4s, void *k4, void *k4s, void *v4,
                    void *v4s, void *stream);

/* Bytes of device workspace thrift_select needs (the pooled fp32 means of Q
 * and K, their norms, the largest K norm of each KV head):
 * 4 * (nb * (d + 1) * B * (Hq + Hkv) + B * Hkv), e.g. 42270752 bytes
 * (40.3 MiB) for B = 1, Hq = 32, Hkv = 8, N = 131072, d = 128.  Returns 0
 * for an invalid shape. */
size_t thrift_select_workspace_bytes(const thrift_shape *s);

/* int32 entries of the traversal-list array: B * Hq * nb(nb+1)/2 (causal) or
 * B * Hq * nb * nb.  Returns 0 for an invalid shape. */
int64_t thrift_list_entries(const thrift_shape *s);

/*
 * Step 2 -- select ("ThriftAttention: Selective Mixed Precision for
 * Long-Context FP4 Attention", abstract: a fast heuristic marks the few
 * important query-key block pairs that stay in FP16).
 *
 * Heuristic: each 64-row block of q16 (per query head) and k16 (per KV head)
 * is mean-pooled (exact sum, one rounding to fp32); a block pair (i, j) is
 * scored by the fp64 dot product of the two means, accumulated in channel
 * order.  Per (b, h_q, query block i), with n_valid = i + 1 (causal) or nb,
 * ppm = llround(frac * 1e6) and forced blocks F = {0, i}:
 *   ppm == 0:  no FP16 blocks;
 *   else:      budget k = min(n_valid, max(|F|, ceil(ppm * n_valid / 1e6)));
 *              FP16 list = F plus the k - |F| best other blocks by
 *              (score descending, block index ascending).
 * The FP4 list is every other valid block.  (The library ranks by fp32
 * chains of the same products and recomputes the fp64 chain of every block
 * whose fp32 score lies within the fp32 chains' error bound of the cut-off:
 * the lists are those of the fp64 ranking, bit for bit.)
 *
 * frac in [0, 1].  Outputs:
 *   idx [B,Hq, rows]: row i starts at i(i+1)/2 (causal) or i*nb and holds the
 *        FP16 list ascending followed by the FP4 list ascending;
 *   n16 [B,Hq,nb]: length of each FP16 list.
 * workspace: device buffer of at least thrift_select_workspace_bytes(s)
 * bytes (contents on return: the pooled means, Q first then K, then their
 * norms; with frac 0 nothing is written).
 * Errors: THRIFT_EINVAL (pointer, frac), THRIFT_EWORKSPACE.
 */
int thrift_select(const thrift_shape *s, double frac, const void *q16, const void *k16, int32_t *idx,
                  int32_t *n16, void *workspace, size_t ws_bytes, void *stream);

/*
 * thrift_select with another block score (the heuristic is the method's open
 * risk: the hotpaper.ai summary of "ThriftAttention: Selective Mixed
 * Precision for Long-Context FP4 Attention", section on significance and
 * limits).  score is a thrift_score; THRIFT_SCORE_POOLED_MEAN gives exactly
 * thrift_select's lists.  The budget rule, the forced blocks, the ranking
 * (score descending, lower block index first) and the list layout are those
 * of thrift_select.  Every score is an fp64 chain over the channels in order
 * (products of fp32 means and fp16 values are exact), so the lists are
 * reproducible bit for bit:
 *   MAX_POOLED     sigma(i,j) = max_r sum_c qbar_i[c] k16[64j + r][c];
 *   NORM_WEIGHTED  the pooled score of norm-weighted means: row r of a block
 *                  weighs w_r = sqrt(fma chain of x_rc^2 over c), the mean is
 *                  (fma chain over r of w_r x_rc) / (sum over r of w_r),
 *                  rounded to fp32 (0 for an all-zero block);
 *   BLOCK_MAX      sigma(i,j) = max over the 64 x 64 row pairs of q . k (64^2
 *                  times the dot products of the pooled score: a comparator).
 * workspace: thrift_select_workspace_bytes(s) bytes (the means).
 * Errors: those of thrift_select, THRIFT_EINVAL for an unknown score.
 */
int thrift_select_ex(const thrift_shape *s, double frac, int score, const void *q16, const void *k16, int32_t *idx,
                     int32_t *n16, void *workspace, size_t ws_bytes, void *stream);

/*
 * The block scores thrift_select_ex ranks, without the selection: scores
 * (fp32, thrift_list_entries(s) entries) receives sigma(i, j) rounded to fp32
 * for every valid block pair, at the list layout's positions (row i at
 * i(i+1)/2 causal or i*nb, entry j).  For studies of the heuristic.
 * Errors: as thrift_select_ex.
 */
int thrift_block_scores(const thrift_shape *s, int score, const void *q16, const void *k16, float *scores,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * thrift_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same lists, bit for bit, with no workspace argument.  The pooled means
 * go to a static device array inside the library (64 MiB per GPU, held
 * until the process ends); the call itself allocates nothing.  Limit:
 * thrift_select_workspace_bytes(s) must not exceed 64 MiB (e.g. B = 1,
 * Hq = 32, Hkv = 8, d = 128 up to N = 208064),
 * else THRIFT_EWORKSPACE and nothing is launched.  The GPU is the stream's
 * (the current device for the default stream).  Every call on one GPU
 * shares that array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialized by the caller.
 * Errors: those of thrift_select, THRIFT_EWORKSPACE beyond the limit.
 */
int thrift_select_noalloc(const thrift_shape *s, double frac, const void *q16, const void *k16, int32_t *idx,
                          int32_t *n16, void *stream);

/*
 * Step 3 -- fused mixed-precision attention (same abstract: the marked
 * blocks run in FP16, every other block in 4-bit, and one online softmax
 * combines the two into a single output).
 *
 * For query row t of (b, h) in block i, every valid key (causal: key <= t)
 * of a block on the row's FP16 list is scored in FP16 (fp32 accumulation)
 * and every key of a block on its FP4 list from the MXFP4 codes.  With
 * c = fl32(sm_scale * log2(e)) (sm_scale <= 0 means 1/sqrt(d)), x = score * c,
 * an integer running max M = ceil(max x) and p = 2^(x - M):
 *   l   = sum of p over all valid keys;
 *   FP16 blocks add fp16(p) * v16 to the accumulator;
 *   FP4 blocks re-quantize p to MXFP4 per aligned 32-key group and add the
 *   MXFP4 product with v4;
 *   out = acc / l;  lse = (M + log2 l) * ln 2 (natural-log LSE of the scaled
 *   scores).
 * out [B,Hq,N,d] of out_dtype (THRIFT_F32, THRIFT_F16 or THRIFT_BF16);
 * lse [B,Hq,N] fp32, may be NULL.  idx/n16 come from thrift_select with the
 * same shape, or follow its layout: each row's FP16 list holds distinct
 * blocks in ascending order; an entry outside [0, n_valid) is skipped, and
 * an n16 above n_valid counts as n_valid.
 * workspace: device buffer of at least thrift_attn_workspace_bytes(s) bytes,
 * 16-byte aligned, owned by the caller; on return it holds each row's
 * partial softmax state after its FP16 blocks (no meaning for the caller).
 * Calls sharing one workspace must not overlap in time.
 * Errors: THRIFT_EINVAL (pointer, dtype, sm_scale), THRIFT_EWORKSPACE.
 */
int thrift_attn_fwd(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                    const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                    const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype,
                    float *lse, void *workspace, size_t ws_bytes, void *stream);

/* thrift_attn_fwd under the other reading of the online-softmax row sum
 * ("ThriftAttention: Selective Mixed Precision for Long-Context FP4
 * Attention", abstract: one online softmax merges both paths; the pages do
 * not say which weights the denominator adds): here l adds the weights the
 * P.V products actually use, fp16(p) on FP16 tiles and the dequantized
 * MXFP4 code of p on FP4 tiles, so every output row is a convex combination
 * of V rows with exactly those weights (V = 1 gives O = 1).  On FP4 tiles the
 * sum comes from one extra scaled MFMA against E2M1 ones instead of a VALU
 * add per score.  Arguments, layouts, ownership, workspace and errors are
 * those of thrift_attn_fwd; lse = (M + log2 l) ln 2 with this l. */
int thrift_attn_fwd_wsum(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                         const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                         const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype,
                         float *lse, void *workspace, size_t ws_bytes, void *stream);

/* thrift_attn_fwd (rowsum 0), thrift_attn_fwd_wsum (rowsum 1), or (rowsum 2)
 * the weights reading with an exp-free FP4 path: on FP4 tiles P's group
 * exponent is the MX rule applied to the group's largest score,
 * e = floor(x_max - M) - 2, and each key's E2M1 code is the nearest-even
 * rounding of 2^floor(y) (1 + frac y), y = x - M - e, a piecewise-linear
 * stand-in for 2^y (equal at integers, at most 6.1% above in between), so
 * no exponential is taken there; the row sum adds the dequantized codes as
 * in rowsum 1.  With an optional timing hook: events, when not NULL, points at four hipEvent_t
 * the caller created (as void *); they are recorded on `stream` before the
 * FP16-tile kernel, between it and the FP4-tile kernel launches (two for a
 * GQA group of odd size: its head pairs, then its last head), between those
 * and the overflow-redo launches, and after them, so the caller can time
 * each phase with hipEventElapsedTime.  Errors: those of thrift_attn_fwd, THRIFT_EINVAL
 * for a rowsum outside 0..2, THRIFT_EHIP if an event cannot be recorded. */
int thrift_attn_fwd_ex(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                       const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                       const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype,
                       float *lse, void *workspace, size_t ws_bytes, void *stream, int rowsum,
                       void *const *events);

/* Bytes of device workspace thrift_attn_fwd (and thrift_attn_fwd_wsum) needs
 * for shape s (0 if s is invalid): B * Hq * N/64 * (2 * 64 * (d/2 + 2) + 1) * 4,
 * e.g. 2214854656 bytes (2.06 GiB) for B = 1, Hq = 32, N = 131072, d = 128. */
size_t thrift_attn_workspace_bytes(const thrift_shape *s);

/* Static string naming a status code. */
const char *thrift_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* THRIFT_H */
