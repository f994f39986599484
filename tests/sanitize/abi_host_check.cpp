// Host-side paths of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer (built with -fsanitize on the host pass only; no GPU needed): the
// workspace size queries over many shapes, the CHMC rank over shapes and
// budgets, fp16 rounding, status strings, the kernel-timing hooks without
// launches, and every entry point's argument checks, which must reject a bad
// call before anything touches the device. Exits non-zero on the first
// mismatch; the sanitizers abort on the first finding.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gptq.h"

static int g_fail = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

int main() {
  void* F = reinterpret_cast<void*>(0x10000);  // never dereferenced
  const int64_t shapes[][2] = {{1, 1},       {37, 129},     {576, 576},    {896, 4864},
                               {4864, 896},  {2048, 5632},  {4096, 14336}, {8192, 28672},
                               {0, 10},      {10, 0},       {1, 1 << 20},  {(int64_t)1 << 26, 4}};
  // workspace queries: no overflow, monotone where they must be
  for (auto& s : shapes) {
    for (int gs : {16, 32, 64, 128, 100}) {
      const size_t q = gptq_quantize_workspace_bytes(s[0], s[1], gs);
      if (s[0] > 0 && s[1] > 0 && gs != 100) EXPECT(q >= (size_t)(s[0] * s[1]));
      else EXPECT(q == 0);
    }
    const size_t p = gptq_prepare_workspace_bytes(s[1]);
    if (s[1] > 0 && s[1] <= 1 << 16) EXPECT(p >= (size_t)(8 * s[1] * s[1]));
    (void)gptq_hessian_workspace_bytes(s[1], s[0]);
    (void)gptq_hessian_split8_workspace_bytes(s[1], s[0]);
    for (int r : {0, 1, 64, 65})
      (void)gptq_chmc_workspace_bytes(s[0], s[1], r);
    for (int b = 1; b <= 9; ++b)
      for (int gs : {16, 32, 64, 128, 0})
        for (double bpw : {0.0, 4.0, 4.2875, 8.0, 1e9}) {
          const int r = gptq_chmc_rank(s[0], s[1], b, gs, bpw);
          EXPECT(r >= 0 && r <= 64);
        }
  }
  EXPECT(gptq_chmc_rank(576, 576, 4, 128, 4.2875) == 2);

  // fp16 rounding: every binary16 value survives the round trip, ties go to
  // even, overflow goes to infinity
  std::vector<double> in;
  for (uint32_t h = 0; h < 0x7c00u; ++h) {
    const int e = (int)(h >> 10), m = (int)(h & 0x3ff);
    const double v = e == 0 ? std::ldexp((double)m, -24) : std::ldexp((double)(1024 + m), e - 25);
    in.push_back(v);
    in.push_back(-v);
  }
  std::vector<uint16_t> out(in.size());
  EXPECT(gptq_fp16_round_host(in.data(), out.data(), (int64_t)in.size()) == GPTQ_OK);
  for (size_t k = 0; k < in.size(); k += 2) {
    EXPECT(out[k] == (uint16_t)(k / 2));
    EXPECT(out[k + 1] == (uint16_t)(0x8000u | (k / 2)));
  }
  const double ties[] = {1.0 + std::ldexp(1.0, -11), 1.0 + 3 * std::ldexp(1.0, -11), 65520.0, 1e300};
  uint16_t t[4];
  EXPECT(gptq_fp16_round_host(ties, t, 4) == GPTQ_OK);
  EXPECT(t[0] == 0x3c00 && t[1] == 0x3c02 && t[2] == 0x7c00 && t[3] == 0x7c00);
  EXPECT(gptq_fp16_round_host(nullptr, t, 1) == GPTQ_EINVAL);
  EXPECT(gptq_fp16_round_host(ties, t, -1) == GPTQ_EINVAL);

  for (int s = -1; s < 8; ++s) EXPECT(std::strlen(gptq_status_string((gptq_status)s)) > 0);
  EXPECT(gptq_version() == 1);
  EXPECT(std::strlen(gptq_last_error_string()) > 0);

  // kernel-timing hooks with nothing recorded
  const int nk = gptq_profile_kernel_count();
  EXPECT(nk > 0 && nk <= 32);
  for (int k = -1; k <= nk; ++k) {
    const char* n = gptq_profile_kernel_name(k);
    EXPECT((k >= 0 && k < nk) ? (n && *n) : n == nullptr);
  }
  std::vector<double> ms(nk, -1.0);
  std::vector<int64_t> cnt(nk, -1);
  EXPECT(gptq_profile_enable(0xffffffffu) == GPTQ_OK);
  EXPECT(gptq_profile_read(ms.data(), cnt.data()) == GPTQ_OK);
  EXPECT(gptq_profile_enable(0) == GPTQ_OK);
  for (int k = 0; k < nk; ++k) EXPECT(ms[k] == 0.0 && cnt[k] == 0);
  EXPECT(gptq_profile_read(nullptr, cnt.data()) == GPTQ_EINVAL);

  // argument checks: every call below is invalid and must return before any
  // HIP call
  double* S = static_cast<double*>(F);
  const float* X = static_cast<const float*>(F);
  EXPECT(gptq_hessian_accumulate(nullptr, 8, X, 4, 8, 0, nullptr, 0, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(S, -1, X, 4, 8, 0, nullptr, 0, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(S, 8, X, 4, 7, 0, nullptr, 0, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_hessian_accumulate(S, 8, X, 4, 8, 0x100u, nullptr, 0, nullptr) == GPTQ_EINVAL);
  int32_t* perm = static_cast<int32_t*>(F);
  float* U = static_cast<float*>(F);
  EXPECT(gptq_prepare_hinv(S, -1, 10, 0.01, 0, perm, U, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(S, 0, 10, 0.01, 0, perm, U, F, 1 << 30, nullptr) == GPTQ_OK);
  EXPECT(gptq_prepare_hinv(S, 8, 10, 0.01, 3u | 8u, perm, U, F, 1 << 30, nullptr) ==
         GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(S, 8, 0, 0.01, 0, perm, U, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(S, 8, 10, -1.0, 0, perm, U, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(S, 8, 10, NAN, 0, perm, U, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_prepare_hinv(S, 8, 10, 0.01, 0, perm, U, nullptr, 0, nullptr) ==
         GPTQ_EWORKSPACE);
  const uint16_t* W = static_cast<const uint16_t*>(F);
  uint8_t* codes = static_cast<uint8_t*>(F);
  uint16_t* sz = static_cast<uint16_t*>(F);
  double* loss = static_cast<double*>(F);
  for (int bits : {1, 9})
    EXPECT(gptq_quantize_layer(W, 4, 8, 8, U, nullptr, bits, 16, 0, codes, sz, sz, nullptr, loss,
                               F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(W, 4, 8, 8, U, nullptr, 4, 24, 0, codes, sz, sz, nullptr, loss, F,
                             1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(W, 4, 8, 7, U, nullptr, 4, 16, 0, codes, sz, sz, nullptr, loss, F,
                             1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_quantize_layer(W, 4, 8, 8, U, nullptr, 4, 16, 0, codes, sz, sz, nullptr, loss,
                             nullptr, 0, nullptr) == GPTQ_EWORKSPACE);
  EXPECT(gptq_quantize_layer_noalloc(W, 9728, 896, 896, U, nullptr, 4, 128, 0, codes, sz, sz,
                                     nullptr, loss, nullptr) == GPTQ_EWORKSPACE);
  EXPECT(gptq_quantize_layer_noalloc(W, 4, 8, 8, U, nullptr, 1, 16, 0, codes, sz, sz, nullptr,
                                     loss, nullptr) == GPTQ_EINVAL);
  uint8_t* mask = static_cast<uint8_t*>(F);
  uint64_t nout = 0;
  double alpha = 0.0;
  EXPECT(gptq_quantize_layer_ssqr(W, 4, 8, 8, U, nullptr, 4, 16, 0, 0.0, codes, sz, sz, nullptr,
                                  loss, mask, sz, &nout, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_ssqr_search(W, 4, 8, 8, U, nullptr, 4, 16, 0, 0.01, 61, 0.1, 1.0, &alpha, codes, sz,
                          sz, nullptr, loss, mask, sz, &nout, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  int64_t nnz = 0;
  EXPECT(gptq_ssqr_outliers_csr(mask, sz, 4, 8, nullptr, perm, sz, 3, 0, &nnz, nullptr) ==
         GPTQ_EINVAL);
  EXPECT(gptq_ssqr_outliers_csr(mask, sz, -1, 8, static_cast<int64_t*>(F), perm, sz, 3, 0, &nnz,
                                nullptr) == GPTQ_EINVAL);
  int16_t* lv = static_cast<int16_t*>(F);
  double bpw = 0.0;
  EXPECT(gptq_quantize_layer_hptq(W, 4, 8, 8, U, nullptr, 4, 16, 0, 17.0, lv, sz, sz, nullptr,
                                  loss, &bpw, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_hptq_search(W, 4, 8, 8, U, nullptr, 4, 16, 0, -1.0, 12, 0.1, 1.0, &alpha, lv, sz,
                          sz, nullptr, loss, &bpw, F, 1 << 30, nullptr) == GPTQ_EINVAL);
  const double* om = static_cast<const double*>(F);
  uint16_t* AB = static_cast<uint16_t*>(F);
  EXPECT(gptq_chmc_layer(W, 64, 128, 128, S, 100, U, nullptr, om, 65, 4, 64, 0, AB, AB, codes,
                         sz, sz, loss, F, (size_t)1 << 40, nullptr, nullptr) == GPTQ_EINVAL);
  EXPECT(gptq_chmc_layer(W, 64, 128, 128, S, 100, U, nullptr, om, 2, 4, 64, 0, AB, AB, codes,
                         sz, sz, loss, nullptr, 0, nullptr, nullptr) == GPTQ_EWORKSPACE);
  EXPECT(gptq_workspace_status(nullptr, nullptr) == GPTQ_EINVAL);

  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
