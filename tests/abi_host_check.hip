// Host-side checks of libspecverify's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py builds and runs it):
// argument validation of every entry point, workspace sizes over a grid of shapes up to the
// int32 limits, the refusals that come before any launch, status strings and the host
// analytics.  Every call here returns before any HIP runtime call or kernel launch, so the
// program needs no GPU; the addresses it passes for device buffers are never dereferenced.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spec_verify.h"

static int g_failures = 0;
static int g_checks = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    ++g_checks;                                                        \
    if (!(cond)) {                                                     \
      std::printf("FAILED (line %d): %s\n", __LINE__, #cond);         \
      ++g_failures;                                                    \
    }                                                                  \
  } while (0)

namespace {

// Stand-ins for device buffers: aligned, never dereferenced on the host.
void* const kDev = reinterpret_cast<void*>(uintptr_t{1} << 20);
const int32_t* const kTok = static_cast<const int32_t*>(kDev);
const float* const kUni = static_cast<const float*>(kDev);
int32_t* const kOutI = static_cast<int32_t*>(kDev);
float* const kOutF = static_cast<float*>(kDev);

sv_sampling samp(float t, int k, float p, float l, float d) { return sv_sampling{t, k, p, l, d}; }

int verify(const void* tgt, sv_dtype dt, int B, int K, int V, int draft_rows,
           const sv_sampling* p, size_t ws_bytes, int32_t* out_n = kOutI) {
  return spec_verify(tgt, kDev, dt, B, K, V, draft_rows, kTok, kUni, p, kOutI, out_n, kOutF,
                     kOutF, kOutF, kDev, ws_bytes, nullptr);
}

void workspace_sizes() {
  const int Bs[] = {1, 7, 256, 65536, INT_MAX};
  const int Ks[] = {0, 1, 7, 64, 1 << 20, INT_MAX};
  const int Vs[] = {1, 2, 31, 16384, 256000, 1 << 24, INT_MAX};
  const sv_sampling modes[] = {
      samp(1.0f, 0, 1.0f, 1.0f, 0.0f),    samp(0.7f, 50, 1.0f, 1.0f, 0.0f),
      samp(0.7f, 300, 1.0f, 1.0f, 0.0f),  samp(1.0f, 0, 0.95f, 1.0f, 0.0f),
      samp(0.7f, 256, 0.9f, 1.0f, 0.0f),  samp(0.0f, 0, 1.0f, 1.0f, 0.0f),
      samp(0.7f, 50, 1.0f, 1.0f, 0.5f),   samp(1.0f, 0, 1.0f, 0.1f, 0.0f)};
  for (int B : Bs)
    for (int K : Ks)
      for (int V : Vs)
        for (const sv_sampling& m : modes)
          for (sv_dtype dt : {SV_DTYPE_F32, SV_DTYPE_BF16}) {
            const size_t n = spec_verify_workspace_size(B, K, V, dt, &m);
            // rows B (2K + 1) must fit int32: otherwise the size is 0 (invalid)
            const long long rows = (long long)B * (2LL * K + 1);
            if (rows > INT_MAX) EXPECT(n == 0);
            if (B == 7 && K == 7 && V == 16384) EXPECT(n > 0);
            (void)spec_sample_workspace_size(B, V, dt, &m);
          }
  for (int B : Bs)
    for (int V : Vs)
      for (int N : {1, 2, 64, 256, 1 << 20, INT_MAX})
        for (sv_dtype dt : {SV_DTYPE_F32, SV_DTYPE_BF16}) (void)spec_verify_tree_workspace_size(B, N, V, dt);
  const sv_sampling ok = samp(1.0f, 0, 1.0f, 1.0f, 0.0f);
  EXPECT(spec_verify_workspace_size(0, 1, 100, SV_DTYPE_F32, &ok) == 0);
  EXPECT(spec_verify_workspace_size(1, -1, 100, SV_DTYPE_F32, &ok) == 0);
  EXPECT(spec_verify_workspace_size(1, 1, 0, SV_DTYPE_F32, &ok) == 0);
  EXPECT(spec_verify_workspace_size(1, 1, 100, (sv_dtype)7, &ok) == 0);
  EXPECT(spec_verify_workspace_size(1, 1, 100, SV_DTYPE_F32, nullptr) == 0);
  EXPECT(spec_verify_tree_workspace_size(0, 4, 100, SV_DTYPE_F32) == 0);
  EXPECT(spec_verify_tree_workspace_size(2, 0, 100, SV_DTYPE_F32) == 0);
}

void verify_arguments() {
  const sv_sampling ok = samp(1.0f, 0, 1.0f, 1.0f, 0.0f);
  const size_t big = (size_t)1 << 40;
  // sampling parameters out of range
  const float nan = std::nanf(""), inf = INFINITY;
  const sv_sampling bad[] = {
      samp(-1.0f, 0, 1.0f, 1.0f, 0.0f), samp(nan, 0, 1.0f, 1.0f, 0.0f),
      samp(inf, 0, 1.0f, 1.0f, 0.0f),   samp(1.0f, -1, 1.0f, 1.0f, 0.0f),
      samp(1.0f, 0, 0.0f, 1.0f, 0.0f),  samp(1.0f, 0, 1.5f, 1.0f, 0.0f),
      samp(1.0f, 0, nan, 1.0f, 0.0f),   samp(1.0f, 0, 1.0f, 0.0f, 0.0f),
      samp(1.0f, 0, 1.0f, 1.5f, 0.0f),  samp(1.0f, 0, 1.0f, nan, 0.0f),
      samp(1.0f, 0, 1.0f, 1.0f, -1.0f), samp(1.0f, 0, 1.0f, 1.0f, inf),
      samp(1.0f, 0, 1.0f, 1.0f, nan),
      samp(0.7f, 50, 1.0f, 0.5f, 0.5f),  // mentored decoding needs lenience 1
      samp(0.7f, 0, 1.0f, 1.0f, 0.5f),   // ... and a compact top-k when sampled
      samp(0.7f, 300, 1.0f, 1.0f, 0.5f)};
  for (const sv_sampling& p : bad) {
    EXPECT(verify(kDev, SV_DTYPE_F32, 4, 3, 1000, 3, &p, big) == SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_workspace_size(4, 3, 1000, SV_DTYPE_F32, &p) == 0);
  }
  // sizes, pointers, dtype
  EXPECT(verify(kDev, SV_DTYPE_F32, 0, 3, 1000, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, 4, -1, 1000, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, 4, 3, 0, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, 4, 3, 1000, 5, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, 4, 3, 1000, 2, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, INT_MAX, 3, 1000, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, (sv_dtype)2, 4, 3, 1000, 3, &ok, big) == SV_ERR_UNSUPPORTED_DTYPE);
  EXPECT(verify(nullptr, SV_DTYPE_F32, 4, 3, 1000, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, 4, 3, 1000, 3, nullptr, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(kDev, SV_DTYPE_F32, 4, 3, 1000, 3, &ok, big, nullptr) == SV_ERR_INVALID_ARG);
  const char* base = static_cast<const char*>(kDev);
  EXPECT(verify(base + 1, SV_DTYPE_BF16, 4, 3, 1000, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(verify(base + 2, SV_DTYPE_F32, 4, 3, 1000, 3, &ok, big) == SV_ERR_INVALID_ARG);
  EXPECT(spec_verify(kDev, nullptr, SV_DTYPE_F32, 4, 3, 1000, 3, kTok, kUni, &ok, kOutI, kOutI,
                     nullptr, nullptr, nullptr, kDev, big, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_verify(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, nullptr, kUni, &ok, kOutI, kOutI,
                     nullptr, nullptr, nullptr, kDev, big, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_verify(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, kTok, nullptr, &ok, kOutI, kOutI,
                     nullptr, nullptr, nullptr, kDev, big, nullptr) == SV_ERR_INVALID_ARG);
  // a workspace one byte short, every sampling mode and both dtypes
  const sv_sampling modes[] = {ok, samp(0.7f, 50, 1.0f, 1.0f, 0.0f),
                               samp(0.7f, 300, 0.9f, 1.0f, 0.0f), samp(1.0f, 0, 0.95f, 1.0f, 0.0f),
                               samp(0.0f, 0, 1.0f, 1.0f, 0.0f), samp(0.7f, 50, 1.0f, 1.0f, 0.3f)};
  for (const sv_sampling& m : modes)
    for (sv_dtype dt : {SV_DTYPE_F32, SV_DTYPE_BF16}) {
      const size_t need = spec_verify_workspace_size(4, 3, 50000, dt, &m);
      EXPECT(need > 0);
      EXPECT(verify(kDev, dt, 4, 3, 50000, 3, &m, need - 1) == SV_ERR_WORKSPACE_TOO_SMALL);
      EXPECT(verify(kDev, dt, 4, 3, 50000, 3, &m, 0) == SV_ERR_WORKSPACE_TOO_SMALL);
    }
  // the no-allocation variant refuses a problem beyond its built-in scratch before any lookup
  const sv_sampling topp = samp(1.0f, 0, 0.95f, 1.0f, 0.0f);
  EXPECT(spec_verify_workspace_size(128, 3, 256000, SV_DTYPE_F32, &topp) >
         SPEC_VERIFY_NOALLOC_SCRATCH_BYTES);
  EXPECT(spec_verify_noalloc(kDev, kDev, SV_DTYPE_F32, 128, 3, 256000, 3, kTok, kUni, &topp,
                             kOutI, kOutI, kOutF, kOutF, kOutF, nullptr) ==
         SV_ERR_SCRATCH_TOO_SMALL);
  EXPECT(spec_verify_noalloc(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, kTok, kUni, &ok, kOutI,
                             nullptr, kOutF, kOutF, kOutF, nullptr) == SV_ERR_INVALID_ARG);
  // the profiled variant needs at least two events
  hipEvent_t ev[2] = {nullptr, nullptr};
  EXPECT(spec_verify_profiled(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, kTok, kUni, &ok, kOutI,
                              kOutI, nullptr, nullptr, nullptr, kDev, big, nullptr, ev, 1) ==
         SV_ERR_INVALID_ARG);
}

void other_entry_points() {
  const sv_sampling ok = samp(1.0f, 0, 1.0f, 1.0f, 0.0f);
  const sv_sampling topk = samp(0.7f, 50, 1.0f, 1.0f, 0.0f);
  const size_t big = (size_t)1 << 40;
  // rates: K >= 1, out_beta given, no mentored decoding
  EXPECT(spec_acceptance_rate(kDev, kDev, SV_DTYPE_F32, 4, 0, 1000, 0, &ok, kOutF, kDev, big,
                              nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_acceptance_rate(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, &ok, nullptr, kDev, big,
                              nullptr) == SV_ERR_INVALID_ARG);
  const sv_sampling ment = samp(0.7f, 50, 1.0f, 1.0f, 0.5f);
  EXPECT(spec_acceptance_rate(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, &ment, kOutF, kDev, big,
                              nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_acceptance_rate(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, &ok, kOutF, kDev, 1,
                              nullptr) == SV_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(spec_verify_rates(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, 3, kTok, kUni, &ok, kOutI,
                           kOutI, kOutF, kOutF, kOutF, nullptr, kDev, big, nullptr) ==
         SV_ERR_INVALID_ARG);
  // presampled: needs a compact top-k, K >= 1 and a large enough sample workspace
  EXPECT(spec_verify_presampled(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, kTok, kUni, &ok, kOutI,
                                kOutI, kOutF, kOutF, kOutF, kDev, big, kDev, big, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_verify_presampled(kDev, kDev, SV_DTYPE_F32, 4, 0, 1000, kTok, kUni, &topk, kOutI,
                                kOutI, kOutF, kOutF, kOutF, kDev, big, kDev, big, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_verify_presampled(kDev, kDev, SV_DTYPE_F32, 4, 3, 1000, kTok, kUni, &topk, kOutI,
                                kOutI, kOutF, kOutF, kOutF, kDev, 1, kDev, big, nullptr) ==
         SV_ERR_WORKSPACE_TOO_SMALL);
  // spec_sample
  EXPECT(spec_sample(kDev, SV_DTYPE_F32, 0, 1000, kUni, &ok, kOutI, kDev, big, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_sample(kDev, SV_DTYPE_F32, 4, 1000, nullptr, &ok, kOutI, kDev, big, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_sample(kDev, SV_DTYPE_F32, 4, 1000, kUni, &ok, kOutI, kDev, 1, nullptr) ==
         SV_ERR_WORKSPACE_TOO_SMALL);
  // tree verification
  EXPECT(spec_verify_tree(kDev, SV_DTYPE_F32, 0, 8, 1000, kTok, kTok, 3, kOutI, kOutI, nullptr,
                          kDev, big, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_verify_tree(kDev, SV_DTYPE_F32, 2, 8, 1000, kTok, kTok, -1, kOutI, kOutI, nullptr,
                          kDev, big, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_verify_tree(kDev, SV_DTYPE_F32, 2, 8, 1000, nullptr, kTok, 3, kOutI, kOutI,
                          nullptr, kDev, big, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_verify_tree(kDev, SV_DTYPE_F32, 2, 8, 1000, kTok, kTok, 3, kOutI, kOutI, nullptr,
                          kDev, 0, nullptr) == SV_ERR_WORKSPACE_TOO_SMALL);
  // tree building: 1 <= M <= 128, 1 <= L <= 32, 1 <= N <= 256
  int32_t* o = kOutI;
  uint8_t* mask = static_cast<uint8_t*>(kDev);
  EXPECT(spec_build_tree(kTok, 2, 0, 8, 16, o, o, o, o, o, mask, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_build_tree(kTok, 2, 129, 8, 16, o, o, o, o, o, mask, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_build_tree(kTok, 2, 8, 33, 16, o, o, o, o, o, mask, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_build_tree(kTok, 2, 8, 8, 257, o, o, o, o, o, mask, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_build_tree(kTok, 0, 8, 8, 16, o, o, o, o, o, mask, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_build_tree(nullptr, 2, 8, 8, 16, o, o, o, o, o, mask, nullptr) ==
         SV_ERR_INVALID_ARG);
  // device uniforms
  EXPECT(spec_philox_uniform(1, 2, 3, -1, kOutF, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_philox_uniform(1, 2, 3, (int64_t{1} << 40) + 1, kOutF, nullptr) ==
         SV_ERR_INVALID_ARG);
  EXPECT(spec_philox_uniform(1, 2, 3, 8, nullptr, nullptr) == SV_ERR_INVALID_ARG);
  EXPECT(spec_philox_uniform(1, 2, 3, 0, nullptr, nullptr) == SV_OK);
}

void strings_and_analytics() {
  for (int s = -3; s <= 8; ++s) {
    const char* str = spec_verify_status_string(s);
    EXPECT(str != nullptr && std::strlen(str) > 0);
  }
  EXPECT(std::fabs(spec_expected_tokens(0.5, 4) - 1.9375) < 1e-15);
  EXPECT(spec_expected_tokens(1.0, 4) == 5.0);
  EXPECT(spec_expected_tokens(0.0, 4) == 1.0);
  EXPECT(std::isnan(spec_expected_tokens(-0.1, 4)));
  EXPECT(std::isnan(spec_expected_tokens(1.1, 4)));
  EXPECT(std::isnan(spec_expected_tokens(std::nan(""), 4)));
  EXPECT(std::isnan(spec_expected_tokens(0.5, -1)));
  EXPECT(std::fabs(spec_walltime_speedup(0.5, 4, 0.0) - 1.9375) < 1e-15);
  EXPECT(std::isnan(spec_walltime_speedup(0.5, 4, -1.0)));
  EXPECT(std::isnan(spec_ops_factor(0.5, 4, -1.0)));
  EXPECT(spec_optimal_gamma(0.8, 0.05, 16) >= 1);
  EXPECT(spec_optimal_gamma(0.8, 0.05, 0) == -1);
  EXPECT(spec_optimal_gamma(1.5, 0.05, 8) == -1);
  for (int g : {0, 1, 7, 64, 1 << 20, INT_MAX})
    for (double a : {0.0, 1e-300, 0.3, 0.999999, 1.0}) {
      (void)spec_expected_tokens(a, g);
      (void)spec_walltime_speedup(a, g, 0.1);
      (void)spec_ops_factor(a, g, 0.1);
    }
  (void)spec_optimal_gamma(0.9, 0.01, 4096);
}

}  // namespace

int main() {
  workspace_sizes();
  verify_arguments();
  other_entry_points();
  strings_and_analytics();
  std::printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
