/*
 * CPU oracle for the ThriftAttention prefill hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct fp64 C.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no source with the GPU library (fp16_long_context_amd/csrc)
 * and neither side includes or links the other.
 *
 * What it follows ("ThriftAttention: Selective Mixed Precision for
 * Long-Context FP4 Attention", abstract):
 *   - stage 1: a cheap heuristic marks the few query-key block pairs that
 *     matter most;
 *   - stage 2: those run at FP16 precision, every other block in
 *     block-scaled 4-bit, and one online softmax combines the two kinds of
 *     block into the result.
 * The abstract leaves the heuristic, the 4-bit format, the block size, the
 * budget rule and the handling of P open.  The readings used here are:
 *   - 4-bit format: OCP MXFP4 (E2M1 elements, one E8M0 scale per 32
 *     elements); scale exponent floor(log2 amax) - 2, elements rounded to
 *     nearest-even on the E2M1 grid and saturated to +-6; codes taken from the
 *     FP16 copy; Q and K grouped along the head dimension, V along tokens.
 *   - blocks: 64 query rows x 64 key rows.
 *   - heuristic: mean-pool every 64-row block of Q (per query head) and K
 *     (per KV head) and score a block pair by the fp64 dot product of the two
 *     means; per query block keep the first and the diagonal key block and
 *     top up with the best-scoring blocks to ceil(frac * valid blocks) in
 *     total (ties -> lower block index); frac = 0 keeps nothing.
 *   - softmax state: one row max held as an integer M = ceil(max x) in log2
 *     units (so rescaling is by exact powers of two, which leaves MXFP4
 *     re-quantization of P unchanged), p = fl32(2^(x - M)), row sum l of the
 *     unquantized p over both paths.
 *   - FP16 path: P rounded to fp16 (nearest-even) before P.V.
 *   - FP4 path: P re-quantized to MXFP4 per aligned 32-key group before P.V.
 *   - GQA: query head h reads KV head floor(h * Hkv / Hq).
 *
 * Arithmetic is fp64 throughout; the exact quantities (pooled sums, FP4 group
 * dot products) are exact in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL -1

/* ------------------------------------------------------------------ */
/* Scalar formats                                                       */
/* ------------------------------------------------------------------ */

/* IEEE binary16 bits -> exact double. */
static double half_bits_to_double(uint16_t h) {
  int sign = h >> 15, ex = (h >> 10) & 31, man = h & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24);
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man + 1024), ex - 25);
  return sign ? -v : v;
}

/* bfloat16 bits -> exact double (bf16 is the top half of a binary32). */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* double -> IEEE binary16 bits, round to nearest, ties to even.  Magnitudes
 * that round past 65504 become infinity. */
static uint16_t double_to_half_bits(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return 0x7e00;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) -> floor(log2 a) = e2 - 1 */
  int E = e2 - 1;
  if (E < -14) {
    /* subnormal range: a value is m * 2^-24 */
    double m = rint(a * 2.0 * 8388608.0); /* a * 2^24 (default rounding mode is nearest-even) */
    return (uint16_t)(sign | (uint16_t)m); /* m == 1024 is the smallest normal */
  }
  double m = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* E2M1 magnitudes indexed by the 3-bit magnitude code (OCP MX v1.0). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static double e2m1_value(int code) {
  double v = E2M1_MAG[code & 7];
  return (code & 8) ? -v : v;
}

/* Nearest E2M1 magnitude code for y >= 0 (already divided by the scale),
 * ties to the even code, saturating at 6. */
static int e2m1_magnitude_code(double y) {
  if (y <= 0.25) return 0;
  if (y < 0.75) return 1;
  if (y <= 1.25) return 2;
  if (y < 1.75) return 3;
  if (y <= 2.5) return 4;
  if (y < 3.5) return 5;
  if (y <= 5.0) return 6;
  return 7;
}

/* MXFP4-encode one group of n values: scale exponent e = floor(log2 amax) - 2
 * clamped to [-127, 127] (-127 for an all-zero group), element code = sign bit
 * | nearest-even E2M1 code of |v| * 2^-e.  Returns the E8M0 byte e + 127. */
static uint8_t mx_encode_group(const double *v, int n, uint8_t *codes) {
  double amax = 0.0;
  for (int i = 0; i < n; i++)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  int e;
  if (amax == 0.0) {
    e = -127;
  } else {
    int e2;
    frexp(amax, &e2);
    e = (e2 - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
  }
  double inv = ldexp(1.0, -e);
  for (int i = 0; i < n; i++)
    codes[i] = (uint8_t)(e2m1_magnitude_code(fabs(v[i]) * inv) | (signbit(v[i]) ? 8 : 0));
  return (uint8_t)(e + 127);
}

static double e8m0_value(uint8_t s) { return ldexp(1.0, (int)s - 127); }

/*
 * The exp-free encoding of one 32-key group of P (the other row-sum reading's
 * cheap FP4 path): x[e] are the keys' scores in log2 units (-inf for a masked
 * key), M the row's integer running max.  The group exponent follows the MX
 * rule applied to the largest p = 2^(xmax - M) without forming it:
 * e = clamp(floor(xmax - M) - 2, -127, 127).  Each key's code is the E2M1
 * rounding (nearest-even, saturating) of a piecewise-linear stand-in for
 * 2^y, y = x - M - e: 2^floor(y) * (1 + y - floor(y)), which agrees with 2^y
 * at integers and is at most 6.1% above it in between; y <= -127 gives 0.
 * No exponential is taken.  Returns the scale byte.
 */
static uint8_t log_encode_group(const double *x, double M, uint8_t *codes) {
  double xmax = -INFINITY;
  for (int k = 0; k < 32; k++)
    if (x[k] > xmax) xmax = x[k];
  int e = (xmax == -INFINITY) ? -127 : (int)floor(xmax - M) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  for (int k = 0; k < 32; k++) {
    double y = x[k] - M - e, z = 0.0;
    if (y > -127.0) {
      double f = floor(y);
      z = ldexp(1.0 + (y - f), (int)f);
    }
    codes[k] = (uint8_t)e2m1_magnitude_code(z);
  }
  return (uint8_t)(e + 127);
}

/* packed nibble accessors: element 2j in the low nibble of byte j */
static int nib(const uint8_t *p, int64_t i) { return (p[i >> 1] >> ((i & 1) * 4)) & 15; }

/* Threads an OpenMP region of the oracle uses (1 without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Exported scalar helpers (used by the oracle's own pin tests)         */
/* ------------------------------------------------------------------ */

void oracle_to_fp16(const uint16_t *in, int in_dtype, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++)
    out[i] = double_to_half_bits(in_dtype == 1 ? bf16_bits_to_double(in[i]) : half_bits_to_double(in[i]));
}

/* Encode ngroups groups of 32 doubles; codes are written one per byte (unpacked). */
void oracle_mx_encode(const double *v, int64_t ngroups, uint8_t *codes, uint8_t *scales) {
  for (int64_t g = 0; g < ngroups; g++) scales[g] = mx_encode_group(v + 32 * g, 32, codes + 32 * g);
}

/* ------------------------------------------------------------------ */
/* Step 1: FP16 copies and MXFP4 codes                                  */
/* ------------------------------------------------------------------ */
/*
 * Layouts (row-major, contiguous):
 *   q [B,Hq,N,d], k/v [B,Hkv,N,d] input bits (in_dtype 0 = fp16, 1 = bf16)
 *   q16 [B,Hq,N,d], k16/v16 [B,Hkv,N,d] fp16 bits
 *   q4 [B,Hq,N,d/2], q4s [B,Hq,N,d/32]; k4/k4s likewise with Hkv
 *   v4 [B,Hkv,d,N/2], v4s [B,Hkv,d,N/32] (groups of 32 tokens per channel)
 */
int oracle_quantize(int B, int Hq, int Hkv, int N, int d, int in_dtype, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, uint16_t *q16, uint16_t *k16, uint16_t *v16, uint8_t *q4, uint8_t *q4s,
                    uint8_t *k4, uint8_t *k4s, uint8_t *v4, uint8_t *v4s) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d % 32 || N % 32) return ORC_EINVAL;
  int64_t nq = (int64_t)B * Hq * N * d, nk = (int64_t)B * Hkv * N * d;
  oracle_to_fp16(q, in_dtype, q16, nq);
  oracle_to_fp16(k, in_dtype, k16, nk);
  oracle_to_fp16(v, in_dtype, v16, nk);

  /* Q and K: groups of 32 consecutive channels of one row */
  for (int which = 0; which < 2; which++) {
    const uint16_t *x16 = which ? k16 : q16;
    uint8_t *x4 = which ? k4 : q4, *x4s = which ? k4s : q4s;
    int64_t rows = (int64_t)B * (which ? Hkv : Hq) * N;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
      double g[32];
      uint8_t c[32];
      for (int m = 0; m < d / 32; m++) {
        for (int i = 0; i < 32; i++) g[i] = half_bits_to_double(x16[r * d + 32 * m + i]);
        x4s[r * (d / 32) + m] = mx_encode_group(g, 32, c);
        for (int i = 0; i < 16; i++) x4[r * (d / 2) + 16 * m + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
      }
    }
  }
  /* V: groups of 32 consecutive tokens of one channel */
  int64_t heads = (int64_t)B * Hkv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < heads; bh++) {
    for (int ch = 0; ch < d; ch++) {
      double g[32];
      uint8_t c[32];
      for (int t0 = 0; t0 < N; t0 += 32) {
        for (int i = 0; i < 32; i++) g[i] = half_bits_to_double(v16[(bh * N + t0 + i) * d + ch]);
        int64_t row = bh * d + ch;
        v4s[row * (N / 32) + t0 / 32] = mx_encode_group(g, 32, c);
        for (int i = 0; i < 16; i++) v4[row * (N / 2) + t0 / 2 + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
      }
    }
  }
  return ORC_OK;
}

/* The exp-free group encoding above, for ngroups groups of 32 scores (log2
 * units) against the integer max M: codes [ngroups, 32], scale bytes. */
void oracle_log_encode(const double *x, int64_t ngroups, double M, uint8_t *codes, uint8_t *scales) {
  for (int64_t g = 0; g < ngroups; g++) scales[g] = log_encode_group(x + 32 * g, M, codes + 32 * g);
}

/* ------------------------------------------------------------------ */
/* Step 2: block heuristic                                              */
/* ------------------------------------------------------------------ */

/* Mean of each 64-row block of x16 [BH, N, d]: exact fp64 sum, one division by
 * 64 (exact), one rounding to fp32.  out [BH, N/64, d]. */
void oracle_pool(const uint16_t *x16, int64_t BH, int N, int d, float *out) {
  int nb = N / 64;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < BH; bh++)
    for (int i = 0; i < nb; i++)
      for (int c = 0; c < d; c++) {
        double s = 0.0;
        for (int r = 0; r < 64; r++) s += half_bits_to_double(x16[(bh * N + 64 * i + r) * d + c]);
        out[(bh * nb + i) * d + c] = (float)(s / 64.0);
      }
}

/* Block score: dot product of two pooled means, summed in channel order in fp64. */
static double block_score(const float *a, const float *b, int d) {
  double s = 0.0;
  for (int c = 0; c < d; c++) s += (double)a[c] * (double)b[c];
  return s;
}

/*
 * Other block scores (the heuristic is the method's open risk: the
 * hotpaper.ai summary of "ThriftAttention: Selective Mixed Precision for
 * Long-Context FP4 Attention", section on significance and limits).  Each
 * replaces the pooled-mean score; the budget rule, forced blocks and ranking
 * stay the same.  All sums are fp64 and sequential in the order stated, so the
 * GPU reproduces them bit for bit.
 *   SCORE_MAX_POOLED   max over the 64 key rows r of block j of the dot
 *                      product of the query block's pooled mean with k_r
 *                      (channel order): one strong key is not averaged away.
 *   SCORE_NORM_WEIGHTED  dot product of norm-weighted block means: row r of a
 *                      block weighs w_r = its L2 norm (sqrt of the channel-order
 *                      sum of squares); mean_c = (sum_r w_r x_rc) / (sum_r w_r),
 *                      both sums in row order, rounded once to fp32 (0 for an
 *                      all-zero block).
 *   SCORE_BLOCK_MAX    max over every (query row, key row) pair of the two
 *                      blocks of their exact dot product: the block's largest
 *                      score, which needs all of Q K^T (a comparator, not a
 *                      cheap heuristic).
 */
enum { SCORE_POOLED = 0, SCORE_MAX_POOLED = 1, SCORE_NORM_WEIGHTED = 2, SCORE_BLOCK_MAX = 3 };

void oracle_normw_pool(const uint16_t *x16, int64_t BH, int N, int d, float *out) {
  int nb = N / 64;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < BH; bh++)
    for (int i = 0; i < nb; i++) {
      const uint16_t *blk = x16 + (bh * N + 64 * (int64_t)i) * d;
      double w[64], wsum = 0.0;
      for (int r = 0; r < 64; r++) {
        double ss = 0.0;
        for (int c = 0; c < d; c++) {
          double x = half_bits_to_double(blk[r * d + c]);
          ss = fma(x, x, ss);
        }
        w[r] = sqrt(ss);
        wsum += w[r];
      }
      for (int c = 0; c < d; c++) {
        double acc = 0.0;
        for (int r = 0; r < 64; r++) acc = fma(w[r], half_bits_to_double(blk[r * d + c]), acc);
        out[(bh * nb + i) * d + c] = wsum > 0.0 ? (float)(acc / wsum) : 0.0f;
      }
    }
}

/* max over the 64 key rows of block kblk of (query mean . k_r) */
static double score_max_pooled(const float *q, const uint16_t *kblk, int d) {
  double best = -INFINITY;
  for (int r = 0; r < 64; r++) {
    double s = 0.0;
    for (int c = 0; c < d; c++) s += (double)q[c] * half_bits_to_double(kblk[r * d + c]);
    if (s > best) best = s;
  }
  return best;
}

/* max over the 64 x 64 row pairs of (q_a . k_r) */
static double score_block_max(const uint16_t *qblk, const uint16_t *kblk, int d) {
  double best = -INFINITY;
  for (int a = 0; a < 64; a++)
    for (int r = 0; r < 64; r++) {
      double s = 0.0;
      for (int c = 0; c < d; c++) s += half_bits_to_double(qblk[a * d + c]) * half_bits_to_double(kblk[r * d + c]);
      if (s > best) best = s;
    }
  return best;
}

int64_t oracle_list_entries(int B, int Hq, int N, int causal) {
  int64_t nb = N / 64;
  int64_t per = causal ? nb * (nb + 1) / 2 : nb * nb;
  return (int64_t)B * Hq * per;
}

/* Number of key blocks that block-row i may attend to. */
static int valid_blocks(int i, int nb, int causal) { return causal ? i + 1 : nb; }
static int64_t row_offset(int64_t i, int64_t nb, int causal) { return causal ? i * (i + 1) / 2 : i * nb; }

typedef struct {
  double s;
  int j;
} scored_t;

static int by_score_desc_then_index(const void *pa, const void *pb) {
  const scored_t *a = pa, *b = pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

/*
 * Per (b, h_q, query block i): n_valid key blocks; ppm = llround(frac * 1e6);
 * budget k = min(n_valid, max(|F|, ceil(ppm * n_valid / 1e6))) with forced set
 * F = {0, i}; the FP16 list is F plus the k - |F| best remaining blocks by
 * (score descending, index ascending); ppm = 0 gives an empty FP16 list.  The
 * FP4 list is every other valid block.  Row i of idx (offset i(i+1)/2 causal,
 * i*nb otherwise) holds the FP16 list ascending then the FP4 list ascending;
 * n16[b,h,i] = FP16 list length.  scores (nullable) receives sigma(i,j) for
 * valid pairs in the same row layout.
 */
int oracle_select_kind(int kind, int B, int Hq, int Hkv, int N, int d, int causal, double frac,
                       const uint16_t *q16, const uint16_t *k16, int32_t *idx, int32_t *n16, float *qbar,
                       float *kbar, double *scores) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N % 64 || !(frac >= 0.0 && frac <= 1.0)) return ORC_EINVAL;
  if (kind < SCORE_POOLED || kind > SCORE_BLOCK_MAX) return ORC_EINVAL;
  int nb = N / 64;
  if (kind == SCORE_NORM_WEIGHTED) {
    oracle_normw_pool(q16, (int64_t)B * Hq, N, d, qbar);
    oracle_normw_pool(k16, (int64_t)B * Hkv, N, d, kbar);
  } else {
    oracle_pool(q16, (int64_t)B * Hq, N, d, qbar);
    oracle_pool(k16, (int64_t)B * Hkv, N, d, kbar);
  }
  long long ppm = llround(frac * 1e6);
  int64_t per = causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
#pragma omp parallel for collapse(3) schedule(dynamic, 4)
  for (int b = 0; b < B; b++)
    for (int h = 0; h < Hq; h++)
      for (int i = 0; i < nb; i++) {
        int g = (int)((int64_t)h * Hkv / Hq);
        int nv = valid_blocks(i, nb, causal);
        const float *qi = qbar + (((int64_t)b * Hq + h) * nb + i) * d;
        int64_t off = ((int64_t)b * Hq + h) * per + row_offset(i, nb, causal);
        scored_t *cand = malloc(sizeof(scored_t) * (size_t)nv);
        char *in16 = calloc((size_t)nv, 1);
        for (int j = 0; j < nv; j++) {
          double s;
          const uint16_t *kblk = k16 + (((int64_t)b * Hkv + g) * N + 64 * (int64_t)j) * d;
          if (kind == SCORE_MAX_POOLED)
            s = score_max_pooled(qi, kblk, d);
          else if (kind == SCORE_BLOCK_MAX)
            s = score_block_max(q16 + (((int64_t)b * Hq + h) * N + 64 * (int64_t)i) * d, kblk, d);
          else
            s = block_score(qi, kbar + (((int64_t)b * Hkv + g) * nb + j) * d, d);
          if (scores) scores[off + j] = s;
          cand[j].s = s;
          cand[j].j = j;
        }
        int count16 = 0;
        if (ppm > 0) {
          in16[0] = 1;
          in16[i] = 1;
          int nforced = (i == 0) ? 1 : 2;
          long long want = (ppm * nv + 999999) / 1000000;
          long long kk = want > nforced ? want : nforced;
          if (kk > nv) kk = nv;
          /* rank the non-forced blocks */
          int nc = 0;
          for (int j = 0; j < nv; j++)
            if (!in16[j]) cand[nc++] = cand[j];
          qsort(cand, (size_t)nc, sizeof(scored_t), by_score_desc_then_index);
          for (long long t = 0; t < kk - nforced; t++) in16[cand[t].j] = 1;
          count16 = (int)kk;
        }
        int w = 0;
        for (int j = 0; j < nv; j++)
          if (in16[j]) idx[off + w++] = j;
        for (int j = 0; j < nv; j++)
          if (!in16[j]) idx[off + w++] = j;
        n16[((int64_t)b * Hq + h) * nb + i] = count16;
        free(cand);
        free(in16);
      }
  return ORC_OK;
}

/* The library's default heuristic: pooled-mean scores. */
int oracle_select(int B, int Hq, int Hkv, int N, int d, int causal, double frac, const uint16_t *q16,
                  const uint16_t *k16, int32_t *idx, int32_t *n16, float *qbar, float *kbar, double *scores) {
  return oracle_select_kind(SCORE_POOLED, B, Hq, Hkv, N, d, causal, frac, q16, k16, idx, n16, qbar, kbar, scores);
}

/* ------------------------------------------------------------------ */
/* Step 3: mixed-precision attention, one output row at a time          */
/* ------------------------------------------------------------------ */
/*
 * rows[r] = ((b * Hq) + h) * N + t selects the output rows to compute.
 * blk_keep (nullable, length N/64): only key blocks with blk_keep[j] != 0
 * take part (used to check that a split online-softmax merge equals one
 * pass).  Per row the outputs are acc[d] (unnormalised), l, M, and
 * out[d] = acc / l, lse = (M + log2 l) * ln 2 (natural-log LSE of the scaled
 * scores).  A row with no participating key gets M = -inf, l = 0, acc = 0,
 * out = 0, lse = -inf.
 *
 * rowsum selects what the row sum l adds up:
 *   0  the unquantized p of every key (the row sum of the online softmax
 *      before any rounding of P; the reading the main path follows);
 *   1  the weights the P.V products actually use: fp16(p) on FP16 tiles and
 *      the dequantized MXFP4 code of p on FP4 tiles, so the output is a
 *      convex combination of V rows with exactly those weights (the
 *      alternative reading: normalisation by the quantized weights);
 *   2  as 1, with the FP4 tiles' P codes taken without an exponential
 *      (log_encode_group): the exp-free FP4 path this reading allows.
 * acc and (for rowsum 1) l take the same terms in the same order.
 *
 * v16 here is [B,Hkv,N,d] (token-major).
 */
int oracle_attn_rows(int B, int Hq, int Hkv, int N, int d, int causal, float sm_scale, const uint16_t *q16,
                     const uint16_t *k16, const uint16_t *v16, const uint8_t *q4, const uint8_t *q4s,
                     const uint8_t *k4, const uint8_t *k4s, const uint8_t *v4, const uint8_t *v4s,
                     const int32_t *idx, const int32_t *n16, const int64_t *rows, int64_t nrows,
                     const uint8_t *blk_keep, double *out, double *lse, double *acc_out, double *l_out,
                     double *m_out, int rowsum) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N % 64 || d % 32 || rowsum < 0 || rowsum > 2) return ORC_EINVAL;
  int nb = N / 64;
  int64_t per = causal ? (int64_t)nb * (nb + 1) / 2 : (int64_t)nb * nb;
  /* score scale in log2 units: c = fl32(sm_scale * log2(e)), sm_scale <= 0 -> fl32(1/sqrt(d)) */
  float sm = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)d));
  double c = (double)(float)((double)sm * 1.4426950408889634074);
  int ok = 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; r++) {
    int64_t rid = rows[r];
    int64_t t = rid % N, bh = rid / N;
    int64_t h = bh % Hq, b = bh / Hq;
    int64_t g = h * Hkv / Hq;
    int64_t kvh = b * Hkv + g;
    int i = (int)(t / 64);
    int nv = valid_blocks(i, nb, causal);
    int64_t off = bh * per + row_offset(i, nb, causal);
    int cnt16 = n16[bh * nb + i];
    /* precision of every key block of this row: 16, 4 or 0 (not attended) */
    char *prec = calloc((size_t)nb, 1);
    for (int e = 0; e < nv; e++) {
      int j = idx[off + e];
      if (j < 0 || j >= nv) {
#pragma omp atomic write
        ok = 0;
        continue;
      }
      prec[j] = (e < cnt16) ? 16 : 4;
    }
    if (blk_keep)
      for (int j = 0; j < nb; j++)
        if (!blk_keep[j]) prec[j] = 0;
    int64_t nkeys = (int64_t)nb * 64;
    double *x = malloc(sizeof(double) * (size_t)nkeys);
    char *live = calloc((size_t)nkeys, 1);
    double xmax = -INFINITY;
    const uint16_t *qrow16 = q16 + rid * d;
    const uint8_t *qrow4 = q4 + rid * (d / 2), *qrow4s = q4s + rid * (d / 32);
    /* scores */
    for (int j = 0; j < nb; j++) {
      if (!prec[j]) continue;
      for (int kk = 0; kk < 64; kk++) {
        int64_t key = (int64_t)j * 64 + kk;
        if (causal && key > t) continue;
        int64_t krow = kvh * N + key;
        double s = 0.0;
        if (prec[j] == 16) {
          for (int ch = 0; ch < d; ch++)
            s += half_bits_to_double(qrow16[ch]) * half_bits_to_double(k16[krow * d + ch]);
        } else {
          for (int m = 0; m < d / 32; m++) {
            double gs = 0.0; /* exact: products are multiples of 1/4 bounded by 36 */
            for (int ch = 32 * m; ch < 32 * m + 32; ch++)
              gs += e2m1_value(nib(qrow4, ch)) * e2m1_value(nib(k4 + krow * (d / 2), ch));
            s += e8m0_value(qrow4s[m]) * e8m0_value(k4s[krow * (d / 32) + m]) * gs;
          }
        }
        x[key] = s * c;
        live[key] = 1;
        if (x[key] > xmax) xmax = x[key];
      }
    }
    double *acc = calloc((size_t)d, sizeof(double));
    double l = 0.0, M = -INFINITY;
    if (xmax > -INFINITY) {
      M = ceil(xmax);
      double *p = calloc((size_t)nkeys, sizeof(double));
      for (int64_t key = 0; key < nkeys; key++)
        if (live[key]) {
          p[key] = (double)(float)exp2(x[key] - M);
          if (rowsum == 0) l += p[key];
        }
      for (int j = 0; j < nb; j++) {
        if (prec[j] == 16) {
          for (int kk = 0; kk < 64; kk++) {
            int64_t key = (int64_t)j * 64 + kk;
            if (!live[key]) continue;
            double p16 = half_bits_to_double(double_to_half_bits(p[key]));
            if (rowsum >= 1) l += p16;
            for (int ch = 0; ch < d; ch++) acc[ch] += p16 * half_bits_to_double(v16[(kvh * N + key) * d + ch]);
          }
        } else if (prec[j] == 4) {
          for (int grp = 0; grp < 2; grp++) {
            int64_t k0 = (int64_t)j * 64 + 32 * grp;
            uint8_t pc[32], ps;
            if (rowsum == 2) {
              /* exp-free codes from the scores; masked keys enter as -inf */
              double xg[32];
              for (int e = 0; e < 32; e++) xg[e] = live[k0 + e] ? x[k0 + e] : -INFINITY;
              ps = log_encode_group(xg, M, pc);
            } else {
              /* masked keys enter the group as zeros */
              ps = mx_encode_group(p + k0, 32, pc);
            }
            if (rowsum >= 1) {
              double gw = 0.0; /* exact group sum of the codes' values */
              for (int e = 0; e < 32; e++) gw += e2m1_value(pc[e]);
              l += e8m0_value(ps) * gw;
            }
            for (int ch = 0; ch < d; ch++) {
              const uint8_t *vrow = v4 + (kvh * d + ch) * (N / 2);
              double gs = 0.0; /* exact group sum */
              for (int e = 0; e < 32; e++) gs += e2m1_value(pc[e]) * e2m1_value(nib(vrow, k0 + e));
              acc[ch] += e8m0_value(ps) * e8m0_value(v4s[(kvh * d + ch) * (N / 32) + k0 / 32]) * gs;
            }
          }
        }
      }
      free(p);
    }
    for (int ch = 0; ch < d; ch++) {
      if (out) out[r * d + ch] = l > 0.0 ? acc[ch] / l : 0.0;
      if (acc_out) acc_out[r * d + ch] = acc[ch];
    }
    if (lse) lse[r] = l > 0.0 ? (M + log2(l)) * 0.69314718055994530942 : -INFINITY;
    if (l_out) l_out[r] = l;
    if (m_out) m_out[r] = M;
    free(acc);
    free(x);
    free(live);
    free(prec);
  }
  return ok ? ORC_OK : ORC_EINVAL;
}
