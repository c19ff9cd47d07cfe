// C ABI of libthrift (declared in include/thrift.h): argument validation on
// the host, then launches on the caller's stream.  Validation runs before
// any HIP call, so an invalid call returns without touching the device.
#include <math.h>

#include "../../include/thrift.h"
#include "thrift_internal.h"

using namespace thrift;

namespace {

int check_shape(const thrift_shape *s) {
  if (!s) return THRIFT_EINVAL;
  if (s->B <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->N <= 0 || s->d <= 0 || s->block <= 0) return THRIFT_EINVAL;
  if (s->Hq % s->Hkv != 0) return THRIFT_EINVAL;
  if (s->causal != 0 && s->causal != 1) return THRIFT_EINVAL;
  if (s->d != 64 && s->d != 128) return THRIFT_EUNSUPPORTED;
  if (s->block != 64) return THRIFT_EUNSUPPORTED;
  if (s->N % 64 != 0 || s->N / 64 > kMaxBlocks) return THRIFT_EUNSUPPORTED;
  // one workgroup of up to 256 threads per (b, query head, query block): a
  // launch addresses fewer than 2^32 threads, so B * Hq * N/64 < 2^24
  const int64_t rows = (int64_t)s->B * s->Hq * (s->N / 64);
  if (rows >= (1LL << 24)) return THRIFT_EUNSUPPORTED;
  return THRIFT_OK;
}

bool aligned_ok(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

// Runs launch() with the stream's GPU current (HIP applies the kernels'
// shared-memory attributes and symbol lookups to the current device), then
// makes the caller's device current again.  The default stream (NULL) runs
// on the current device.
template <class F>
int on_stream_device(void *stream, F launch) {
  int cur = 0, dev = 0;
  if (stream) {
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return THRIFT_EHIP;
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return THRIFT_EHIP;
  }
  const hipError_t e = launch();
  if (stream && dev != cur && hipSetDevice(cur) != hipSuccess) return THRIFT_EHIP;
  return e == hipSuccess ? THRIFT_OK : THRIFT_EHIP;
}

}  // namespace

extern "C" {

const char *thrift_status_str(int status) {
  switch (status) {
    case THRIFT_OK: return "ok";
    case THRIFT_EINVAL: return "invalid argument";
    case THRIFT_EUNSUPPORTED: return "unsupported shape";
    case THRIFT_EWORKSPACE: return "workspace missing or too small";
    case THRIFT_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t thrift_select_workspace_bytes(const thrift_shape *s) {
  if (check_shape(s) != THRIFT_OK) return 0;
  return sizeof(float) * select_workspace_floats(s->B, s->Hq, s->Hkv, s->N, s->d);
}

int64_t thrift_list_entries(const thrift_shape *s) {
  if (check_shape(s) != THRIFT_OK) return 0;
  const int64_t nb = s->N / 64;
  return (int64_t)s->B * s->Hq * (s->causal ? nb * (nb + 1) / 2 : nb * nb);
}

int thrift_quantize(const thrift_shape *s, int in_dtype, const void *q, const void *k, const void *v, void *q16,
                    void *k16, void *v16, void *q4, void *q4s, void *k4, void *k4s, void *v4, void *v4s,
                    void *stream) {
  int rc = check_shape(s);
  if (rc != THRIFT_OK) return rc;
  if (in_dtype != THRIFT_F16 && in_dtype != THRIFT_BF16) return THRIFT_EINVAL;
  const void *ptrs[] = {q, k, v, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s};
  for (const void *p : ptrs)
    if (!aligned_ok(p)) return THRIFT_EINVAL;
  QuantArgs a;
  a.q = q; a.k = k; a.v = v;
  a.q16 = (uint16_t *)q16; a.k16 = (uint16_t *)k16; a.v16 = (uint16_t *)v16;
  a.q4 = (uint8_t *)q4; a.q4s = (uint8_t *)q4s; a.k4 = (uint8_t *)k4; a.k4s = (uint8_t *)k4s;
  a.v4 = (uint8_t *)v4; a.v4s = (uint8_t *)v4s;
  a.B = s->B; a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.d = s->d;
  a.bf16 = in_dtype == THRIFT_BF16;
  return on_stream_device(stream, [&] { return launch_quantize(a, (hipStream_t)stream); });
}

int thrift_select(const thrift_shape *s, double frac, const void *q16, const void *k16, int32_t *idx, int32_t *n16,
                  void *workspace, size_t ws_bytes, void *stream) {
  int rc = check_shape(s);
  if (rc != THRIFT_OK) return rc;
  if (!(frac >= 0.0 && frac <= 1.0)) return THRIFT_EINVAL;  // also rejects NaN
  const void *ptrs[] = {q16, k16, idx, n16};
  for (const void *p : ptrs)
    if (!aligned_ok(p)) return THRIFT_EINVAL;
  const size_t need = thrift_select_workspace_bytes(s);
  if (!workspace || ws_bytes < need) return THRIFT_EWORKSPACE;
  if (!aligned_ok(workspace)) return THRIFT_EINVAL;
  SelectArgs a;
  a.q16 = (const uint16_t *)q16; a.k16 = (const uint16_t *)k16;
  a.idx = idx; a.n16 = n16;
  a.B = s->B; a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.d = s->d; a.causal = s->causal;
  select_layout(a, (float *)workspace);
  a.ppm = (int64_t)llround(frac * 1e6);
  return on_stream_device(stream, [&] { return launch_select(a, (hipStream_t)stream); });
}

static int select_args(const thrift_shape *s, double frac, int score, const void *q16, const void *k16,
                       int32_t *idx, int32_t *n16, void *workspace, size_t ws_bytes, SelectArgs &a) {
  int rc = check_shape(s);
  if (rc != THRIFT_OK) return rc;
  if (!(frac >= 0.0 && frac <= 1.0)) return THRIFT_EINVAL;  // also rejects NaN
  if (score < THRIFT_SCORE_POOLED_MEAN || score > THRIFT_SCORE_BLOCK_MAX) return THRIFT_EINVAL;
  const void *ptrs[] = {q16, k16, idx, n16};
  for (const void *p : ptrs)
    if (!aligned_ok(p)) return THRIFT_EINVAL;
  const size_t need = thrift_select_workspace_bytes(s);
  if (!workspace || ws_bytes < need) return THRIFT_EWORKSPACE;
  if (!aligned_ok(workspace)) return THRIFT_EINVAL;
  a.q16 = (const uint16_t *)q16; a.k16 = (const uint16_t *)k16;
  a.idx = idx; a.n16 = n16;
  a.B = s->B; a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.d = s->d; a.causal = s->causal;
  select_layout(a, (float *)workspace);
  a.ppm = (int64_t)llround(frac * 1e6);
  a.kind = score;
  return THRIFT_OK;
}

int thrift_select_ex(const thrift_shape *s, double frac, int score, const void *q16, const void *k16, int32_t *idx,
                     int32_t *n16, void *workspace, size_t ws_bytes, void *stream) {
  SelectArgs a;
  const int rc = select_args(s, frac, score, q16, k16, idx, n16, workspace, ws_bytes, a);
  if (rc != THRIFT_OK) return rc;
  return on_stream_device(stream, [&] { return launch_select(a, (hipStream_t)stream); });
}

int thrift_block_scores(const thrift_shape *s, int score, const void *q16, const void *k16, float *scores,
                        void *workspace, size_t ws_bytes, void *stream) {
  SelectArgs a;
  // n16 is not written: any aligned non-null pointer passes validation
  const int rc = select_args(s, 1.0, score, q16, k16, (int32_t *)scores, (int32_t *)scores, workspace, ws_bytes, a);
  if (rc != THRIFT_OK) return rc;
  return on_stream_device(stream, [&] { return launch_block_scores(a, (hipStream_t)stream); });
}

int thrift_select_noalloc(const thrift_shape *s, double frac, const void *q16, const void *k16, int32_t *idx,
                          int32_t *n16, void *stream) {
  int rc = check_shape(s);
  if (rc != THRIFT_OK) return rc;
  if (!(frac >= 0.0 && frac <= 1.0)) return THRIFT_EINVAL;  // also rejects NaN
  const void *ptrs[] = {q16, k16, idx, n16};
  for (const void *p : ptrs)
    if (!aligned_ok(p)) return THRIFT_EINVAL;
  // the pooled means must fit the library's static scratch array
  if (thrift_select_workspace_bytes(s) > kSelectScratchBytes) return THRIFT_EWORKSPACE;
  SelectArgs a;
  a.q16 = (const uint16_t *)q16; a.k16 = (const uint16_t *)k16;
  a.idx = idx; a.n16 = n16;
  a.qbar = a.kbarT = a.qn = a.kn = a.knmax = nullptr;  // set by the launcher
  a.B = s->B; a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.d = s->d; a.causal = s->causal;
  a.ppm = (int64_t)llround(frac * 1e6);
  return on_stream_device(stream, [&] { return launch_select_scratch(a, (hipStream_t)stream); });
}

size_t thrift_attn_workspace_bytes(const thrift_shape *s) {
  if (check_shape(s) != THRIFT_OK) return 0;
  return attn_workspace_bytes(s->B, s->Hq, s->N, s->d);
}

static int attn_fwd_common(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                           const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                           const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype,
                           float *lse, void *workspace, size_t ws_bytes, void *stream, int rowsum,
                           void *const *events) {
  int rc = check_shape(s);
  if (rc != THRIFT_OK) return rc;
  if (out_dtype != THRIFT_F16 && out_dtype != THRIFT_BF16 && out_dtype != THRIFT_F32) return THRIFT_EINVAL;
  if (!(sm_scale == sm_scale) || isinf(sm_scale)) return THRIFT_EINVAL;
  const void *ptrs[] = {q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, idx, n16, out};
  for (const void *p : ptrs)
    if (!aligned_ok(p)) return THRIFT_EINVAL;
  if (lse && ((uintptr_t)lse & 15u)) return THRIFT_EINVAL;
  if (!workspace || ws_bytes < thrift_attn_workspace_bytes(s)) return THRIFT_EWORKSPACE;
  if (!aligned_ok(workspace)) return THRIFT_EINVAL;
  AttnArgs a;
  a.q16 = (const uint16_t *)q16; a.k16 = (const uint16_t *)k16; a.v16 = (const uint16_t *)v16;
  a.q4 = (const uint8_t *)q4; a.q4s = (const uint8_t *)q4s; a.k4 = (const uint8_t *)k4;
  a.k4s = (const uint8_t *)k4s; a.v4 = (const uint8_t *)v4; a.v4s = (const uint8_t *)v4s;
  a.idx = idx; a.n16 = n16; a.out = out; a.lse = lse; a.ws = (float *)workspace;
  a.B = s->B; a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.d = s->d; a.causal = s->causal;
  a.out_dtype = out_dtype;
  a.rowsum = rowsum;
  // score scale in log2 units, rounded once to fp32
  const float sm = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)s->d));
  a.c = (float)((double)sm * 1.4426950408889634074);
  return on_stream_device(stream, [&] { return launch_attn_fwd(a, (hipStream_t)stream, (hipEvent_t const *)events); });
}

int thrift_attn_fwd(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                    const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                    const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype, float *lse,
                    void *workspace, size_t ws_bytes, void *stream) {
  return attn_fwd_common(s, sm_scale, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, idx, n16, out, out_dtype, lse,
                         workspace, ws_bytes, stream, 0, nullptr);
}

int thrift_attn_fwd_wsum(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                         const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                         const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype,
                         float *lse, void *workspace, size_t ws_bytes, void *stream) {
  return attn_fwd_common(s, sm_scale, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, idx, n16, out, out_dtype, lse,
                         workspace, ws_bytes, stream, 1, nullptr);
}

int thrift_attn_fwd_ex(const thrift_shape *s, float sm_scale, const void *q16, const void *k16, const void *v16,
                       const void *q4, const void *q4s, const void *k4, const void *k4s, const void *v4,
                       const void *v4s, const int32_t *idx, const int32_t *n16, void *out, int out_dtype,
                       float *lse, void *workspace, size_t ws_bytes, void *stream, int rowsum,
                       void *const *events) {
  if (rowsum < 0 || rowsum > 2) return THRIFT_EINVAL;
  return attn_fwd_common(s, sm_scale, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, idx, n16, out, out_dtype, lse,
                         workspace, ws_bytes, stream, rowsum, events);
}

}  // extern "C"
