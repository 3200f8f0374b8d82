// Host-side argument validation and planning of the C ABI, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (see
// tests/test_sanitizers.py).  The kernel launchers are replaced by stubs that
// launch nothing and report a launch error, so no call reaches a GPU: with no
// GPU the calls stop at the device check (FA_ERR_DEVICE), with one at the stub
// (FA_ERR_LAUNCH).  Pointers are fake, aligned or not; none is dereferenced on
// the host.  Exit status 0 = every case returned the expected status.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "fa.h"
#include "fa_kernels.h"

namespace fa {
static int stub_calls = 0;
static hipError_t stub() {
  ++stub_calls;
  return hipErrorInvalidValue;
}
hipError_t launch_bwd_pre(const BwdParams &, int, int, long, hipStream_t) { return stub(); }
hipError_t launch_bwd_dq(const BwdParams &, int, int, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_bwd_dkdv(const BwdParams &, int, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_fwd(const FwdParams &, int, int, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_fwd_split(const FwdParams &, int, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_fwd_combine(const FwdParams &, int, int, long, hipStream_t) { return stub(); }
hipError_t launch_fwd_decode(const FwdParams &, int, int, int, hipStream_t) { return stub(); }
}  // namespace fa

static int failures = 0;
static int checks = 0;

static void expect(int got, int want, const char *what, int line) {
  ++checks;
  if (got != want) {
    std::fprintf(stderr, "FAIL line %d: %s: status %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// a valid call ends at the device check (no GPU) or at the stub (a GPU)
static int g_valid = FA_ERR_DEVICE;
#define VALID(call)                                                            \
  do {                                                                         \
    const int s_ = (call);                                                     \
    expect(s_ == FA_ERR_DEVICE || s_ == FA_ERR_LAUNCH ? g_valid : s_, g_valid, \
           #call, __LINE__);                                                   \
  } while (0)

static void *P = reinterpret_cast<void *>(0x10000);  // aligned, never dereferenced
static void *M = reinterpret_cast<void *>(0x10008);  // misaligned
static const int *L = reinterpret_cast<const int *>(0x20000);
static const int *LM = reinterpret_cast<const int *>(0x20002);

static void forward_cases() {
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = INFINITY;
  VALID(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 64, 0.125f, 0, FA_F16, nullptr));
  VALID(fa_fwd(P, P, P, P, (float *)P, 4, 32, 8192, 128, 0.088f, 1, FA_BF16, nullptr));
  VALID(fa_fwd(P, P, P, P, (float *)P, 1, 1, 16777215, 128, 0.f, 1, FA_BF16, nullptr));
  VALID(fa_fwd(P, P, P, P, (float *)P, 1, 1, 33554431, 64, -1.f, 0, FA_F16, nullptr));
  VALID(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 64, std::numeric_limits<float>::denorm_min(), 0, FA_F16, nullptr));
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 16777216, 128, 0.1f, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, INT_MAX, INT_MAX, INT_MAX, 128, 0.1f, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, INT_MAX, INT_MAX, 1000, 128, 0.1f, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, INT_MIN, 1, 1, 128, 0.1f, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, -1, 1, 128, 0.1f, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, INT_MAX, 0.1f, 1, FA_BF16, nullptr), FA_ERR_HEAD_DIM);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 3, INT_MAX, 0.1f, 1, FA_BF16, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, INT_MIN, 0.1f, 1, FA_BF16, nullptr), FA_ERR_HEAD_DIM);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 96, 0.1f, 1, FA_BF16, nullptr), FA_ERR_HEAD_DIM);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 64, 0.1f, 1, 2, nullptr), FA_ERR_DTYPE);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 64, 0.1f, -1, FA_F16, nullptr), FA_ERR_ARG);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 64, nan, 0, FA_F16, nullptr), FA_ERR_ARG);
  EXPECT(fa_fwd(P, P, P, P, (float *)P, 1, 1, 1, 64, -inf, 0, FA_F16, nullptr), FA_ERR_ARG);
  EXPECT(fa_fwd(nullptr, P, P, P, (float *)P, 1, 1, 1, 64, 0.1f, 0, FA_F16, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd(P, P, P, P, nullptr, 1, 1, 1, 64, 0.1f, 0, FA_F16, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd(P, M, P, P, (float *)P, 1, 1, 1, 64, 0.1f, 0, FA_F16, nullptr), FA_ERR_ALIGN);
  // padded, cross-attention, dropout
  VALID(fa_fwd_padded(P, P, P, P, (float *)P, L, L, 3, 2, 1, 16777215, 128, 0.1f, 1, FA_BF16, nullptr));
  VALID(fa_fwd_padded(P, P, P, P, (float *)P, nullptr, nullptr, 3, 2, 16777215, 1, 128, 0.1f, 0, FA_BF16, nullptr));
  EXPECT(fa_fwd_padded(P, P, P, P, (float *)P, LM, L, 3, 2, 5, 7, 64, 0.1f, 1, FA_F16, nullptr), FA_ERR_ALIGN);
  EXPECT(fa_fwd_padded(P, P, P, P, (float *)P, L, L, 3, 2, 5, 0, 64, 0.1f, 1, FA_F16, nullptr), FA_ERR_SHAPE);
  VALID(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, 0.f, 0, 0, FA_F16, nullptr));
  VALID(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, 255.4f / 256, ~0ULL, ~0u, FA_F16,
                       nullptr));
  EXPECT(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, 1.f, 0, 0, FA_F16, nullptr),
         FA_ERR_ARG);
  EXPECT(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, -0.01f, 0, 0, FA_F16, nullptr),
         FA_ERR_ARG);
  EXPECT(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, nan, 0, 0, FA_F16, nullptr),
         FA_ERR_ARG);
  EXPECT(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, 1e30f, 0, 0, FA_F16, nullptr),
         FA_ERR_ARG);
  EXPECT(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, INFINITY, 0, 0, FA_F16, nullptr),
         FA_ERR_ARG);
  EXPECT(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, 255.5f / 256, 0, 0, FA_F16, nullptr),
         FA_ERR_ARG);
  VALID(fa_fwd_dropout(P, P, P, P, (float *)P, L, L, 3, 2, 5, 7, 64, 0.1f, 1, -0.f, 0, 0, FA_F16, nullptr));
  // split over keys: decode and several rows, extreme key counts
  const int shapes[][5] = {{32, 32, 1, 16384, 128}, {1, 1, 1, 1, 64}, {1, 1, 1, 16777215, 128},
                           {1, 1, 1000, 16777215, 128}, {64, 64, 7, 100, 64}, {1, 1, 16777215, 1, 128}};
  for (const auto &s : shapes) {
    const size_t ws = fa_fwd_splitkv_workspace_size(s[0], s[1], s[2], s[3], s[4]);
    if (ws == 0) {
      std::fprintf(stderr, "FAIL: no split workspace size for %d %d %d %d %d\n", s[0], s[1], s[2], s[3], s[4]);
      ++failures;
      continue;
    }
    VALID(fa_fwd_splitkv(P, P, P, P, (float *)P, nullptr, nullptr, s[0], s[1], s[2], s[3], s[4], 0.1f, 0, FA_BF16,
                         P, ws, nullptr));
    EXPECT(fa_fwd_splitkv(P, P, P, P, (float *)P, nullptr, nullptr, s[0], s[1], s[2], s[3], s[4], 0.1f, 0,
                          FA_BF16, P, ws - 1, nullptr),
           FA_ERR_WORKSPACE);
  }
  EXPECT((int)fa_fwd_splitkv_workspace_size(1, 1, 1, 0, 128), 0);
  EXPECT((int)fa_fwd_splitkv_workspace_size(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128), 0);
  EXPECT(fa_fwd_splitkv(P, P, P, P, (float *)P, nullptr, nullptr, 1, 1, 1, 64, 64, 0.1f, 0, FA_BF16, nullptr, 1 << 20,
                        nullptr),
         FA_ERR_NULL);
}

static void backward_cases() {
  const size_t need = fa_bwd_workspace_size(4, 32, 8192, 128);
  EXPECT(need >= 2u * 4 * 32 * 8192 * 4 ? 0 : 1, 0);
  VALID(fa_bwd(P, P, P, P, P, (float *)P, P, P, P, 4, 32, 8192, 128, 0.088f, 1, FA_BF16, P, need, nullptr));
  EXPECT(fa_bwd(P, P, P, P, P, (float *)P, P, P, P, 4, 32, 8192, 128, 0.088f, 1, FA_BF16, P, need - 1, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(P, P, P, P, P, (float *)P, P, P, P, 4, 32, 8192, 128, 0.088f, 1, FA_BF16, M, need, nullptr),
         FA_ERR_ALIGN);
  EXPECT(fa_bwd(P, P, P, P, P, (float *)P, P, P, P, 4, 32, 8192, 128, INFINITY, 1, FA_BF16, P, need, nullptr),
         FA_ERR_ARG);
  const size_t big = fa_bwd_workspace_size(1, 1, 16777215, 128);
  VALID(fa_bwd(P, P, P, P, P, (float *)P, P, P, P, 1, 1, 16777215, 128, 0.f, 1, FA_F16, P, big, nullptr));
  EXPECT((int)fa_bwd_workspace_size(1, 1, 16777216, 128), 0);
  EXPECT((int)fa_bwd_workspace_size(INT_MAX, INT_MAX, INT_MAX, 64), 0);
  VALID(fa_bwd_preprocess(P, P, (float *)P, 2, 16, 4096, 128, FA_BF16, P, fa_bwd_workspace_size(2, 16, 4096, 128),
                          nullptr));
  VALID(fa_bwd_dq(P, P, P, P, P, 2, 16, 4096, 128, 0.1f, 1, FA_BF16, P, fa_bwd_workspace_size(2, 16, 4096, 128),
                  nullptr));
  VALID(fa_bwd_dkdv(P, P, P, P, P, P, 2, 16, 4096, 64, 0.1f, 0, FA_F16, P, fa_bwd_workspace_size(2, 16, 4096, 64),
                    nullptr));
  VALID(fa_bwd_dq_preprocess(P, P, P, P, P, (float *)P, P, 1, 1, 1, 64, 0.1f, 1, FA_F16, P,
                             fa_bwd_workspace_size(1, 1, 1, 64), nullptr));
  EXPECT(fa_bwd_dq_preprocess(P, P, P, nullptr, P, (float *)P, P, 1, 1, 1, 64, 0.1f, 1, FA_F16, P, 1 << 20, nullptr),
         FA_ERR_NULL);
  // padded and dropout: workspace sized by the query rows
  const size_t wq = fa_bwd_workspace_size(3, 2, 1000, 64);
  VALID(fa_bwd_padded(P, P, P, P, P, (float *)P, P, P, P, L, L, 3, 2, 1000, 16777215 / 2, 64, 0.1f, 1, FA_F16, P, wq,
                      nullptr));
  EXPECT(fa_bwd_padded(P, P, P, P, P, (float *)P, P, P, P, L, L, 3, 2, 1000, 7, 64, 0.1f, 1, FA_F16, P, wq - 1,
                       nullptr),
         FA_ERR_WORKSPACE);
  VALID(fa_bwd_dropout(P, P, P, P, P, (float *)P, P, P, P, nullptr, L, 3, 2, 1000, 7, 64, 0.1f, 1, 0.5f, 123, 9,
                       FA_BF16, P, wq, nullptr));
  EXPECT(fa_bwd_dropout(P, P, P, P, P, (float *)P, P, P, P, nullptr, LM, 3, 2, 1000, 7, 64, 0.1f, 1, 0.5f, 123, 9,
                        FA_BF16, P, wq, nullptr),
         FA_ERR_ALIGN);
  // the no-allocation backward and its row limit
  VALID(fa_bwd_noalloc(P, P, P, P, P, (float *)P, P, P, P, 4, 32, 8192, 128, 0.088f, 1, FA_BF16, nullptr));
  EXPECT(fa_bwd_noalloc(P, P, P, P, P, (float *)P, P, P, P, 4, 32, 32769, 128, 0.088f, 1, FA_BF16, nullptr),
         FA_ERR_SCRATCH);
  EXPECT(fa_bwd_noalloc(P, P, P, P, P, (float *)P, P, P, P, INT_MAX, INT_MAX, 1, 64, 0.1f, 1, FA_BF16, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_bwd_noalloc(P, P, P, P, P, nullptr, P, P, P, 1, 1, 1, 64, 0.1f, 1, FA_BF16, nullptr), FA_ERR_NULL);
}

static void plan_cases() {
  fa_plan_t p;
  const int Ns[] = {1, 2, 127, 128, 129, 8192, 16777215};
  for (int N : Ns)
    for (int d : {64, 128})
      for (int causal = 0; causal < 2; ++causal) {
        if (d == 64 || N <= 16777215) {
          EXPECT(fa_fwd_plan(7, 3, N, d, causal, FA_F16, &p), FA_OK);
          EXPECT(fa_bwd_plan(7, 3, N, d, causal, FA_BF16, &p), FA_OK);
        }
      }
  EXPECT(fa_fwd_plan(INT_MAX, INT_MAX, 1, 64, 0, FA_F16, &p), FA_ERR_SHAPE);
  EXPECT(fa_fwd_plan(INT_MAX, 1, 16777215, 128, 0, FA_F16, &p), FA_ERR_SHAPE);
  EXPECT(fa_bwd_plan(1 << 20, 1 << 10, 256, 128, 0, FA_F16, &p), FA_ERR_SHAPE);
  EXPECT(fa_fwd_plan(1, 1, 1, 64, 0, FA_F16, nullptr), FA_ERR_NULL);
  for (int s = -3; s < 20; ++s) {
    const char *str = fa_status_str(s);
    if (!str || !*str) {
      std::fprintf(stderr, "FAIL: empty status string %d\n", s);
      ++failures;
    }
  }
}

int main() {
  int n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0) g_valid = FA_ERR_LAUNCH;
  (void)hipGetLastError();
  forward_cases();
  backward_cases();
  plan_cases();
  // the same calls in debug mode: plan lines on stderr, no scan (nothing ran)
  setenv("FA_DEBUG", "1", 1);
  forward_cases();
  backward_cases();
  unsetenv("FA_DEBUG");
  if (g_valid == FA_ERR_DEVICE && fa::stub_calls != 0) {
    std::fprintf(stderr, "FAIL: a launcher was reached without a GPU\n");
    ++failures;
  }
  if (failures) {
    std::fprintf(stderr, "%d of %d checks failed\n", failures, checks);
    return 1;
  }
  std::printf("ABI host checks: %d passed (valid calls end with status %d)\n", checks, g_valid);
  return 0;
}
