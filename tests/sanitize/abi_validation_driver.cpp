// Host-only driver of the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitized_host.py).
//
// Every entry point is called over a grid of extreme sizes (negative, zero,
// 2^31 - 1, 2^31, 2^40, 2^56, INT64_MAX, INT64_MIN), bad head dimensions,
// dtypes and scales, and NULL, misaligned and overlapping pointers.  The
// pointers are fake device addresses that nothing dereferences: the kernel
// launchers are replaced at link time (ld --wrap) by stand-ins that record
// the call, check the arguments validation let through, and report a launch
// error, and the scratch array's address lookup returns a fake address, so
// no call reaches a GPU.  The driver fails (exit 1) when a call
// returns a status outside the enum, returns FA_OK for a non-empty problem
// (the launch would have been reached), leaves no message for a failure, or
// lets through arguments the launchers cannot take; the sanitizers abort on
// memory errors and undefined behaviour (signed overflow included).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "fa_api.h"
#include "fa_launch.h"

namespace {

int g_fail = 0;
long g_calls = 0, g_launches = 0;
char g_case[160] = "";   // the arguments of the current call, for messages

void fail(const char* what, const char* detail) {
  if (g_fail < 20) std::fprintf(stderr, "FAIL %s: %s [%s]\n", what, detail, g_case);
  ++g_fail;
}

void check_launch(bool ok, const char* what) {
  ++g_launches;
  if (!ok) fail("launcher received arguments validation should have refused", what);
}

bool fwd_ok(const iofa::FwdArgs& a) {
  return a.Q && a.K && a.V && a.O && a.BH >= 1 && a.N >= 1 && a.Nk >= 1 &&
         (a.d == 64 || a.d == 128) && a.dtype >= 0 && a.dtype <= 2 && std::isfinite(a.scale) &&
         a.BH * a.N < (int64_t(1) << 31) && a.N * a.d < (int64_t(1) << 31) &&
         a.BH * a.Nk < (int64_t(1) << 31) && a.Nk * a.d < (int64_t(1) << 31);
}

}  // namespace

// Link-time stand-ins for the kernel launchers (ld --wrap=<mangled name>).
extern "C" {
hipError_t __wrap__ZN4iofa12launch_fusedERKNS_7FwdArgsE(const iofa::FwdArgs& a) {
  check_launch(fwd_ok(a) && a.LSE, "launch_fused");
  return hipErrorInvalidValue;
}
hipError_t __wrap__ZN4iofa20launch_fused_partialERKNS_7FwdArgsEiPfS3_(const iofa::FwdArgs& a,
                                                                     int splits, float* o,
                                                                     float* l) {
  check_launch(fwd_ok(a) && splits >= 2 && splits <= 64 && o && l, "launch_fused_partial");
  return hipErrorInvalidValue;
}
hipError_t __wrap__ZN4iofa12launch_mergeERKNS_9MergeArgsE(const iofa::MergeArgs& a) {
  check_launch(a.O_part && a.LSE_part && a.O && a.LSE && a.G >= 1 && a.rows >= 1 &&
                   (a.d == 64 || a.d == 128),
               "launch_merge");
  return hipErrorInvalidValue;
}
hipError_t __wrap__ZN4iofa12launch_naiveERKNS_9NaiveArgsE(const iofa::NaiveArgs& a) {
  check_launch(fwd_ok(a.f) && a.S && a.P && a.ldS >= a.f.N && a.f.N <= iofa::kNaiveMaxN,
               "launch_naive");
  return hipErrorInvalidValue;
}
hipError_t __wrap__ZN4iofa14launch_softmaxERKNS_11SoftmaxArgsE(const iofa::SoftmaxArgs& a) {
  bool ok = a.X && a.Y && a.rows >= 1 && a.n >= 1 && a.dtype >= 0 && a.dtype <= 2;
  if (ok) {
    // every grid the call may launch (at most one workgroup per pass-2 piece
    // of every row) stays below 2^31 workgroups, and long rows have a workspace
    const int64_t pieces = (a.n - 1) / iofa::softmax_piece(a.dtype) + 1;
    ok = static_cast<__int128>(a.rows) * pieces < (static_cast<__int128>(1) << 31) &&
         (a.n <= iofa::softmax_chunk(a.dtype) || a.workspace);
  }
  check_launch(ok, "launch_softmax");
  return hipErrorInvalidValue;
}
// Which form a softmax call takes asks the device for its capacity; here it
// only checks what reaches it.
int __wrap__ZN4iofa15softmax_x_readsERKNS_11SoftmaxArgsE(const iofa::SoftmaxArgs& a) {
  ++g_launches;
  if (!(a.rows >= 1 && a.n >= 1 && a.dtype >= 0 && a.dtype <= 2))
    fail("softmax_x_reads received arguments fa_softmax_x_reads should have refused", "");
  return 2;
}
hipError_t __wrap__ZN4iofa10launch_bwdERKNS_7BwdArgsE(const iofa::BwdArgs& a) {
  check_launch(a.Q && a.K && a.V && a.O && a.dO && a.LSE && a.dQ && a.dK && a.dV && a.stats &&
                   a.BH >= 1 && a.N >= 1 && (a.d == 64 || a.d == 128) &&
                   (a.dtype == 1 || a.dtype == 2),
               "launch_bwd");
  return hipErrorInvalidValue;
}
hipError_t __wrap__ZN4iofa15scratch_addressEPPv(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(1) << 50);   // a fake device address
  return hipSuccess;
}
hipError_t __wrap__ZN4iofa10launch_fp8ERKNS_7Fp8ArgsE(const iofa::Fp8Args& a) {
  check_launch(a.Q && a.K && a.V && a.O && a.LSE && a.BH >= 1 && a.N >= 1 &&
                   (a.d == 64 || a.d == 128) && std::isfinite(a.c2) && a.v_scale > 0.f,
               "launch_fp8");
  return hipErrorInvalidValue;
}
}

namespace {

// Fake device addresses 1 TiB apart (never dereferenced).
void* fake(int i, uintptr_t off = 0) {
  return reinterpret_cast<void*>((uintptr_t(1) << 44) * uintptr_t(i + 1) + off);
}

void after(int st, bool empty, const char* what) {
  ++g_calls;
  if (st < 0 || st > FA_ERR_HIP) fail(what, "status outside fa_status");
  if (st == FA_OK && !empty) fail(what, "FA_OK for a non-empty problem (launch not reached)");
  if (st != FA_OK && std::strlen(fa_last_error()) == 0) fail(what, "no message for a failure");
  if (std::strcmp(fa_status_string(st), "unknown status") == 0) fail(what, "status has no name");
}

const int64_t kBig[] = {-1,
                        0,
                        1,
                        3,
                        1000,
                        (int64_t(1) << 31) - 1,
                        int64_t(1) << 31,
                        int64_t(1) << 40,
                        int64_t(1) << 56,
                        std::numeric_limits<int64_t>::max(),
                        std::numeric_limits<int64_t>::min()};
const int64_t kD[] = {64, 128, 0, 96, -64, std::numeric_limits<int64_t>::max()};
const int kDtype[] = {0, 1, 2, 3, -1};
const float kScale[] = {0.125f, -2.f, std::numeric_limits<float>::infinity(),
                        std::numeric_limits<float>::quiet_NaN()};

// Pointer sets: 0 distinct aligned, 1 a NULL output, 2 misaligned, 3 O on Q.
struct Ptrs {
  void *q, *k, *v, *o, *x1, *x2, *x3, *x4, *ws;
  float* lse;
};
Ptrs ptrs(int kind) {
  Ptrs p{fake(0), fake(1), fake(2), fake(3), fake(5), fake(6), fake(7), fake(8), fake(9),
         static_cast<float*>(fake(4))};
  if (kind == 1) p.o = nullptr;
  if (kind == 2) p.k = fake(1, 2);
  if (kind == 3) p.o = p.q;
  return p;
}

bool is_empty(int64_t B, int64_t H, int64_t N) { return B == 0 || H == 0 || N == 0; }

}  // namespace

int main() {
  for (int64_t B : kBig)
    for (int64_t H : kBig)
      for (int64_t N : kBig)
        for (int64_t d : kD)
          for (int dt : kDtype)
            for (float sc : kScale)
              for (int pk = 0; pk < 4; ++pk) {
                const Ptrs p = ptrs(pk);
                std::snprintf(g_case, sizeof(g_case),
                              "B=%lld H=%lld N=%lld d=%lld dtype=%d scale=%g pointers=%d",
                              static_cast<long long>(B), static_cast<long long>(H),
                              static_cast<long long>(N), static_cast<long long>(d), dt,
                              static_cast<double>(sc), pk);
                const bool shape_ok = B >= 0 && H >= 0 && N >= 0 && (d == 64 || d == 128) &&
                                      std::isfinite(sc);
                const bool empty = shape_ok && dt >= 0 && dt <= 2 && is_empty(B, H, N);
                after(fa_fwd(p.q, p.k, p.v, p.o, p.lse, B, H, N, d, sc, dt, nullptr), empty,
                      "fa_fwd");
                after(fa_naive_fwd(p.q, p.k, p.v, p.o, pk == 2 ? nullptr : p.lse, p.x1, p.x2, B,
                                   H, N, d, sc, dt, nullptr),
                      empty, "fa_naive_fwd");
                for (int g : {0, 1, 4, 64, 1000}) {
                  const size_t need = fa_splitkv_workspace_bytes(B, H, N, d, dt, g);
                  (void)fa_splitkv_num_splits(B, H, N, d, dt, g);
                  after(fa_fwd_splitkv(p.q, p.k, p.v, p.o, p.lse, p.ws, need, g, B, H, N, d, sc,
                                       dt, nullptr),
                        empty, "fa_fwd_splitkv");
                }
                for (int g : {0, 1, 4, 64})
                  after(fa_fwd_splitkv_noalloc(p.q, p.k, p.v, p.o, p.lse, g, B, H, N, d, sc, dt,
                                               nullptr),
                        empty, "fa_fwd_splitkv_noalloc");
                const size_t bw = fa_bwd_workspace_bytes(B, H, N);
                after(fa_bwd(p.q, p.k, p.v, p.x1, p.x2, p.lse, p.o, p.x3, p.x4, p.ws, bw, B, H, N,
                             d, sc, dt, nullptr),
                      empty && dt != 0, "fa_bwd");
                // the FP8 call has no dtype; pointers=3 gives it a negative v_scale
                after(fa_fwd_fp8(p.q, p.k, p.v, p.o, p.lse, B, H, N, d, sc, 0.5f, 2.f,
                                 pk == 3 ? -1.f : 1.f, nullptr),
                      shape_ok && is_empty(B, H, N) && pk != 3, "fa_fwd_fp8");
                (void)fa_naive_workspace_bytes(B, H, N, dt);
              }
  // the split-KV forward over queries and keys of different lengths
  for (int64_t B : kBig)
    for (int64_t H : {int64_t(1), int64_t(3)})
      for (int64_t Nq : kBig)
        for (int64_t Nk : kBig)
          for (int64_t d : kD)
            for (int dt : kDtype)
              for (float sc : {0.125f, std::numeric_limits<float>::infinity()})
                for (int pk : {0, 2, 3}) {
                  const Ptrs p = ptrs(pk);
                  std::snprintf(g_case, sizeof(g_case),
                                "qk B=%lld H=%lld Nq=%lld Nk=%lld d=%lld dtype=%d scale=%g "
                                "pointers=%d",
                                static_cast<long long>(B), static_cast<long long>(H),
                                static_cast<long long>(Nq), static_cast<long long>(Nk),
                                static_cast<long long>(d), dt, static_cast<double>(sc), pk);
                  const bool empty = B >= 0 && Nq >= 0 && Nk >= 0 && (d == 64 || d == 128) &&
                                     std::isfinite(sc) && dt >= 0 && dt <= 2 &&
                                     (B == 0 || Nq == 0);
                  for (int g : {0, 4}) {
                    const size_t need = fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, dt, g);
                    (void)fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, dt, g);
                    after(fa_fwd_splitkv_qk(p.q, p.k, p.v, p.o, p.lse, p.ws, need, g, B, H, Nq,
                                            Nk, d, sc, dt, nullptr),
                          empty, "fa_fwd_splitkv_qk");
                  }
                }
  // merge and softmax over their own arguments
  for (int64_t rows : kBig)
    for (int64_t d : kD)
      for (int dt : kDtype)
        for (int g : {-1, 0, 1, 7, 4096, 4097})
          for (int pk = 0; pk < 4; ++pk) {
            const Ptrs p = ptrs(pk);
            std::snprintf(g_case, sizeof(g_case), "rows=%lld d=%lld dtype=%d parts=%d pointers=%d",
                          static_cast<long long>(rows), static_cast<long long>(d), dt, g, pk);
            const bool empty = rows == 0 && dt >= 0 && dt <= 2 && g >= 1 && g <= 4096 &&
                               (d == 64 || d == 128);
            after(fa_merge_partials(static_cast<float*>(p.q), static_cast<float*>(p.k), g, rows,
                                    d, p.o, p.lse, dt, nullptr),
                  empty, "fa_merge_partials");
          }
  for (int64_t rows : kBig)
    for (int64_t n : kBig)
      for (int dt : kDtype)
        for (int pk = 0; pk < 4; ++pk) {
          const Ptrs p = ptrs(pk);
          std::snprintf(g_case, sizeof(g_case), "rows=%lld n=%lld dtype=%d pointers=%d",
                        static_cast<long long>(rows), static_cast<long long>(n), dt, pk);
          const size_t need = fa_softmax_workspace_bytes(rows, n, dt);
          const bool empty = dt >= 0 && dt <= 2 && rows >= 0 && n >= 0 && (rows == 0 || n == 0);
          after(fa_softmax_rows(p.q, pk == 3 ? p.q : p.o, p.lse, rows, n, dt, p.ws, need,
                                nullptr),
                empty, "fa_softmax_rows");
          after(fa_softmax_rows(p.q, p.o, nullptr, rows, n, dt, nullptr, 0, nullptr), empty,
                "fa_softmax_rows (no workspace)");
          const int reads = fa_softmax_x_reads(p.q, p.o, rows, n, dt);
          const bool valid = dt >= 0 && dt <= 2 && rows >= 1 && n >= 1;
          if (reads != (valid ? 2 : 0)) fail("fa_softmax_x_reads", "unexpected result");
        }
  for (int polls : {0, 1, 400, -1, std::numeric_limits<int>::max(), std::numeric_limits<int>::min()})
    (void)fa_softmax_set_wait_limit(polls);
  if (fa_softmax_set_wait_limit(-1) != 400) fail("fa_softmax_set_wait_limit", "default not restored");
  std::printf("calls %ld, launches reached (intercepted) %ld, failures %d\n", g_calls, g_launches,
              g_fail);
  if (g_launches == 0) fail("driver", "no call reached a launcher");
  return g_fail == 0 ? 0 : 1;
}
