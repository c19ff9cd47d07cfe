// The C ABI driven from plain C++ with the HIP runtime only (no Python, no
// torch): quantize -> select -> attention on inputs read from a file, results
// written to a file for comparison with the oracle.
//
// usage: c_abi_check IN OUT
// IN:  int32 B, Hq, Hkv, N, d, causal; double frac; then q [B,Hq,N,d],
//      k [B,Hkv,N,d], v [B,Hkv,N,d] as fp16 bit patterns (uint16).
// OUT: int32 status; then idx (int32, thrift_list_entries), n16 (int32,
//      B*Hq*N/64), out (fp32, B*Hq*N*d), lse (fp32, B*Hq*N).
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "thrift.h"

static int fail(const char *what, int rc) {
  std::fprintf(stderr, "%s failed: %d (%s)\n", what, rc, thrift_status_str(rc));
  return 1;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE *fi = std::fopen(argv[1], "rb");
  if (!fi) return fail("open input", -1);
  int32_t hdr[6];
  double frac;
  if (std::fread(hdr, sizeof hdr, 1, fi) != 1 || std::fread(&frac, sizeof frac, 1, fi) != 1) return fail("read header", -1);
  thrift_shape s{hdr[0], hdr[1], hdr[2], hdr[3], hdr[4], 64, hdr[5]};
  const size_t nq = (size_t)s.B * s.Hq * s.N * s.d, nk = (size_t)s.B * s.Hkv * s.N * s.d;
  std::vector<uint16_t> hq(nq), hk(nk), hv(nk);
  if (std::fread(hq.data(), 2, nq, fi) != nq || std::fread(hk.data(), 2, nk, fi) != nk ||
      std::fread(hv.data(), 2, nk, fi) != nk)
    return fail("read inputs", -1);
  std::fclose(fi);

  const size_t nb = (size_t)s.N / 64, rows = (size_t)s.B * s.Hq * s.N;
  const size_t ents = thrift_list_entries(&s);
  const size_t sws = thrift_select_workspace_bytes(&s), aws = thrift_attn_workspace_bytes(&s);
  if (!ents || !sws || !aws) return fail("shape", THRIFT_EINVAL);

  void *q, *k, *v, *q16, *k16, *v16, *q4, *q4s, *k4, *k4s, *v4, *v4s, *idx, *n16, *out, *lse, *ws, *wa;
  HIP_OK(hipMalloc(&q, nq * 2));
  HIP_OK(hipMalloc(&k, nk * 2));
  HIP_OK(hipMalloc(&v, nk * 2));
  HIP_OK(hipMalloc(&q16, nq * 2));
  HIP_OK(hipMalloc(&k16, nk * 2));
  HIP_OK(hipMalloc(&v16, nk * 2));
  HIP_OK(hipMalloc(&q4, nq / 2));
  HIP_OK(hipMalloc(&q4s, nq / 32));
  HIP_OK(hipMalloc(&k4, nk / 2));
  HIP_OK(hipMalloc(&k4s, nk / 32));
  HIP_OK(hipMalloc(&v4, nk / 2));
  HIP_OK(hipMalloc(&v4s, nk / 32));
  HIP_OK(hipMalloc(&idx, ents * 4));
  HIP_OK(hipMalloc(&n16, (size_t)s.B * s.Hq * nb * 4));
  HIP_OK(hipMalloc(&out, rows * s.d * 4));
  HIP_OK(hipMalloc(&lse, rows * 4));
  HIP_OK(hipMalloc(&ws, sws));
  HIP_OK(hipMalloc(&wa, aws));
  HIP_OK(hipMemcpy(q, hq.data(), nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk.data(), nk * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv.data(), nk * 2, hipMemcpyHostToDevice));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  int rc = thrift_quantize(&s, THRIFT_F16, q, k, v, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, st);
  if (rc) return fail("thrift_quantize", rc);
  rc = thrift_select(&s, frac, q16, k16, (int32_t *)idx, (int32_t *)n16, ws, sws, st);
  if (rc) return fail("thrift_select", rc);
  rc = thrift_attn_fwd(&s, 0.0f, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, (const int32_t *)idx,
                       (const int32_t *)n16, out, THRIFT_F32, (float *)lse, wa, aws, st);
  if (rc) return fail("thrift_attn_fwd", rc);
  HIP_OK(hipStreamSynchronize(st));

  std::vector<int32_t> h_idx(ents), h_n16((size_t)s.B * s.Hq * nb);
  std::vector<float> h_out(rows * s.d), h_lse(rows);
  HIP_OK(hipMemcpy(h_idx.data(), idx, ents * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_n16.data(), n16, h_n16.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_out.data(), out, h_out.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_lse.data(), lse, h_lse.size() * 4, hipMemcpyDeviceToHost));
  FILE *fo = std::fopen(argv[2], "wb");
  if (!fo) return fail("open output", -1);
  const int32_t ok = 0;
  std::fwrite(&ok, 4, 1, fo);
  std::fwrite(h_idx.data(), 4, h_idx.size(), fo);
  std::fwrite(h_n16.data(), 4, h_n16.size(), fo);
  std::fwrite(h_out.data(), 4, h_out.size(), fo);
  std::fwrite(h_lse.data(), 4, h_lse.size(), fo);
  std::fclose(fo);
  for (void *p : {q, k, v, q16, k16, v16, q4, q4s, k4, k4s, v4, v4s, idx, n16, out, lse, ws, wa}) HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(st));
  std::printf("c_abi_check ok: B=%d Hq=%d Hkv=%d N=%d d=%d frac=%g\n", s.B, s.Hq, s.Hkv, s.N, s.d, frac);
  return 0;
}
