// C ABI of the gfx950 exact-attention library: argument validation, error
// reporting and dispatch to the kernel launchers.  Validation touches no HIP
// API, so a call with bad arguments returns its status on any host, with or
// without a GPU.
#include "../../include/fa_api.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "fa_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int elem_bytes(int dtype) {
  switch (dtype) {
    case FA_F32: return 4;
    case FA_F16: return 2;
    case FA_BF16: return 2;
    default: return 0;
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Only for 0 <= n <= kNaiveMaxN (callers check the bound first).
int64_t round_up8(int64_t n) { return (n + 7) / 8 * 8; }

// Ceiling of n / m for n >= 0, m > 0, without overflow for any int64 n.
int64_t ceil_div(int64_t n, int64_t m) { return n / m + (n % m != 0); }

// The product of the factors in size_t, or 0 when it does not fit.
size_t product_or_zero(std::initializer_list<size_t> factors) {
  size_t r = 1;
  for (size_t f : factors)
    if (__builtin_mul_overflow(r, f, &r)) return 0;
  return r;
}

// Sizes within the library's limits -- B * H < 2^31, N * d < 2^31 and
// B * H * N < 2^31 -- evaluated without signed overflow for any int64
// input.  B, H, N >= 1 and d > 0 are the caller's to check first.
bool within_limits(int64_t B, int64_t H, int64_t N, int64_t d) {
  constexpr int64_t kLim = (int64_t(1) << 31) - 1;
  if (B > kLim || H > kLim || B * H > kLim) return false;   // B, H < 2^31: no overflow
  if (N > kLim / d) return false;                            // N * d < 2^31
  return B * H * N <= kLim;                                  // < 2^31 * 2^31: no overflow
}

// Split-KV policy: at most this many key ranges, and enough of them that the
// partial pass has about this many waves (eight per CU on 256 CUs), but,
// when G is chosen automatically, no fewer than kMinKeysPerSplit keys per
// range (shorter ranges spend more on the pipeline's fill and drain and on
// the merge than the extra workgroups win back: B2 H4 N2048 d128 took 33.3
// us unsplit, 34.0 at G = 2 and 36.6 at G = 4, with K and V read from HBM).
constexpr int64_t kMaxSplits = 64;
constexpr int64_t kTargetWaves = 2048;   // 8 per CU on 256 CUs
// With fewer query rows than one query tile (decode) every workgroup is
// bound by its stream of keys and values: one 4-wave workgroup per CU
// measured fastest (B1 H8 Nq1 Nk32768: 29 us against 35 us at 2048 waves;
// B1 H32 Nq1 Nk16384: 44.5 against 44.6 us; K and V not in the last-level
// cache).
constexpr int64_t kTargetWavesShortQueries = 1024;
constexpr int64_t kMinKeysPerSplit = 1024;
// With short queries a range keeps at least kMinKeysShortQueries keys (the
// workgroup's fixed cost against its stream), and more than
// kManySplitsShortQueries ranges only when each keeps kMinKeysManySplits
// (the merge of many partials costs more than the extra workgroups win on
// short ranges).  Measured with K and V read from HBM (bf16, us): B2 H16 Nq1
// Nk1024 d128 G = 8: 9.0 against 12.1 at G = 2; B1 H8 Nq1 Nk4096
// d64 G = 16: 9.0 against 13.7 at G = 4 and 11.1 at G = 32; B1 H8 Nq1
// Nk32768 d128 keeps G = 32.
constexpr int64_t kMinKeysShortQueries = 128;
constexpr int64_t kManySplitsShortQueries = 16;
constexpr int64_t kMinKeysManySplits = 512;
constexpr int kMaxMergeParts = 4096;

struct Region {
  const void* p;
  size_t bytes;
  const char* name;
};

// Shared checks of the forward entry points, for Nq query rows and Nk key
// rows per head (Nq = Nk = N for self-attention).  Returns FA_OK and sets
// *empty when there is nothing to do: no query rows (or B or H zero).
// Queries without keys are refused: their softmax has no terms.
int check_common_qk(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                    bool lse_required, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                    float scale, int dtype, bool* empty) {
  *empty = false;
  const std::string sizes = Nq == Nk ? " N=" + std::to_string(Nq)
                                     : " Nq=" + std::to_string(Nq) + " Nk=" + std::to_string(Nk);
  if (elem_bytes(dtype) == 0)
    return fail(FA_ERR_DTYPE, "dtype " + std::to_string(dtype) + " is not FA_F32, FA_F16 or FA_BF16");
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_SHAPE, "B, H and the sequence lengths must be >= 0 (got B=" +
                                  std::to_string(B) + " H=" + std::to_string(H) + sizes + ")");
  if (d != 64 && d != 128)
    return fail(FA_ERR_HEAD_DIM, "head dimension d must be 64 or 128 (got " + std::to_string(d) + ")");
  if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale must be finite");
  if (B == 0 || H == 0 || Nq == 0) {
    *empty = true;
    return FA_OK;
  }
  if (Nk == 0) return fail(FA_ERR_SHAPE, "query rows need at least one key row (Nk = 0)");
  if (!within_limits(B, H, Nq, d) || !within_limits(B, H, Nk, d))
    return fail(FA_ERR_SHAPE, "B * H, N * d and B * H * N must each be < 2^31 for both lengths "
                              "(got B=" + std::to_string(B) + " H=" + std::to_string(H) + sizes + ")");
  if (!Q || !K || !V || !O) return fail(FA_ERR_NULL, "Q, K, V and O must not be NULL");
  if (lse_required && !LSE) return fail(FA_ERR_NULL, "LSE must not be NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(FA_ERR_ALIGN, "Q, K, V and O must be 16-byte aligned");
  if (LSE && !aligned(LSE, 4)) return fail(FA_ERR_ALIGN, "LSE must be 4-byte aligned");
  return FA_OK;
}

// The same checks for one sequence length (fa_fwd, fa_naive_fwd, ...).
int check_common(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                 bool lse_required, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 int dtype, bool* empty) {
  return check_common_qk(Q, K, V, O, LSE, lse_required, B, H, N, N, d, scale, dtype, empty);
}

int check_aliasing(const Region* in, int nin, const Region* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(out[i].p, out[i].bytes, in[j].p, in[j].bytes))
        return fail(FA_ERR_ALIAS, std::string(out[i].name) + " overlaps input " + in[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i].p, out[i].bytes, out[j].p, out[j].bytes))
        return fail(FA_ERR_ALIAS, std::string(out[i].name) + " overlaps " + out[j].name);
  }
  return FA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
           int64_t H, int64_t N, int64_t d, float scale, int dtype, void* stream) {
  g_last_error.clear();
  bool empty = false;
  int st = check_common(Q, K, V, O, LSE, true, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const size_t tensor = static_cast<size_t>(B * H * N * d) * elem_bytes(dtype);
  const size_t lse = static_cast<size_t>(B * H * N) * sizeof(float);
  const Region in[3] = {{Q, tensor, "Q"}, {K, tensor, "K"}, {V, tensor, "V"}};
  const Region out[2] = {{O, tensor, "O"}, {LSE, lse, "LSE"}};
  st = check_aliasing(in, 3, out, 2);
  if (st != FA_OK) return st;
  if (iofa::fused_workgroups(dtype, B * H, N, 1) >= (int64_t(1) << 31))
    return fail(FA_ERR_SHAPE, "too many workgroups");
  iofa::FwdArgs a{Q, K, V, O, LSE, B * H, N, N, d, scale, dtype, static_cast<hipStream_t>(stream)};
  return hip_status(iofa::launch_fused(a), "fused forward launch");
}

int fa_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
               int64_t H, int64_t N, int64_t d, float scale, float q_scale, float k_scale,
               float v_scale, void* stream) {
  g_last_error.clear();
  const float ts[3] = {q_scale, k_scale, v_scale};
  const char* tn[3] = {"q_scale", "k_scale", "v_scale"};
  for (int i = 0; i < 3; ++i)
    if (!(std::isfinite(ts[i]) && ts[i] > 0.f))
      return fail(FA_ERR_SCALE, std::string(tn[i]) + " must be finite and > 0");
  // shape, head-dimension, scale, pointer and alignment checks of a 16-bit call
  bool empty = false;
  int st = check_common(Q, K, V, O, LSE, true, B, H, N, d, scale, FA_BF16, &empty);
  if (st != FA_OK || empty) return st;
  const double c2 = std::fabs(static_cast<double>(scale)) * q_scale * k_scale * 1.4426950408889634;
  if (!std::isfinite(static_cast<float>(c2)))
    return fail(FA_ERR_SCALE, "|scale| * q_scale * k_scale overflows fp32");
  const size_t codes = static_cast<size_t>(B * H * N * d);
  const size_t lse = static_cast<size_t>(B * H * N) * sizeof(float);
  const Region in[3] = {{Q, codes, "Q"}, {K, codes, "K"}, {V, codes, "V"}};
  const Region out[2] = {{O, codes * 2, "O"}, {LSE, lse, "LSE"}};
  st = check_aliasing(in, 3, out, 2);
  if (st != FA_OK) return st;
  if (iofa::fp8_workgroups(B * H, N) >= (int64_t(1) << 31))
    return fail(FA_ERR_SHAPE, "too many workgroups");
  iofa::Fp8Args a{Q, K, V, O, LSE, B * H, N, d, static_cast<float>(c2), v_scale, scale < 0.f,
                  static_cast<hipStream_t>(stream)};
  return hip_status(iofa::launch_fp8(a), "FP8 forward launch");
}

int fa_splitkv_qk_num_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype,
                             int requested) {
  if (elem_bytes(dtype) == 0 || B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128))
    return 0;
  if (!within_limits(B, H, Nq, d) || !within_limits(B, H, Nk, d)) return 0;
  const int64_t tiles = ceil_div(Nk, iofa::fused_key_tile(dtype, d));
  const int64_t cap = tiles < kMaxSplits ? tiles : kMaxSplits;
  int64_t g = requested;
  if (g <= 0) {
    // enough waves for one full round of the chip
    const int64_t per_split = iofa::fused_waves(dtype, B * H, Nq, 1);
    if (Nq < iofa::fused_query_tile(dtype)) {
      g = (kTargetWavesShortQueries + per_split - 1) / per_split;
      const int64_t longest = Nk / kMinKeysShortQueries;
      if (g > longest) g = longest;
      const int64_t many = std::max(kManySplitsShortQueries, Nk / kMinKeysManySplits);
      if (g > many) g = many;
    } else {
      g = (kTargetWaves + per_split - 1) / per_split;
      const int64_t longest = Nk / kMinKeysPerSplit;
      if (g > longest) g = longest;
    }
  }
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

int fa_splitkv_num_splits(int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int requested) {
  return fa_splitkv_qk_num_splits(B, H, N, N, d, dtype, requested);
}

size_t fa_splitkv_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                     int dtype, int num_splits) {
  const int g = fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, dtype, num_splits);
  if (g <= 1) return 0;
  // g > 1 only for sizes within the limits, so the product fits
  const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(H) * static_cast<size_t>(Nq);
  return static_cast<size_t>(g) * rows * (static_cast<size_t>(d) + 1) * sizeof(float);
}

size_t fa_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                                  int num_splits) {
  return fa_splitkv_qk_workspace_bytes(B, H, N, N, d, dtype, num_splits);
}

int fa_fwd_splitkv_qk(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      void* workspace, size_t workspace_bytes, int num_splits, int64_t B,
                      int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int dtype,
                      void* stream) {
  g_last_error.clear();
  bool empty = false;
  int st = check_common_qk(Q, K, V, O, LSE, true, B, H, Nq, Nk, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const int g = fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, dtype, num_splits);
  const size_t qtensor = static_cast<size_t>(B * H * Nq * d) * elem_bytes(dtype);
  const size_t ktensor = static_cast<size_t>(B * H * Nk * d) * elem_bytes(dtype);
  const size_t lse = static_cast<size_t>(B * H * Nq) * sizeof(float);
  const size_t need = fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, dtype, num_splits);
  if (g > 1) {
    if (!workspace) return fail(FA_ERR_NULL, "workspace must not be NULL when splitting");
    if (!aligned(workspace, 16)) return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_SHAPE, "workspace holds " + std::to_string(workspace_bytes) +
                                    " bytes, the split needs " + std::to_string(need));
  }
  const Region in[3] = {{Q, qtensor, "Q"}, {K, ktensor, "K"}, {V, ktensor, "V"}};
  const Region out[3] = {{O, qtensor, "O"}, {LSE, lse, "LSE"},
                         {workspace, g > 1 ? need : 0, "workspace"}};
  st = check_aliasing(in, 3, out, 3);
  if (st != FA_OK) return st;
  if (iofa::fused_workgroups(dtype, B * H, Nq, g) >= (int64_t(1) << 31) ||
      iofa::merge_workgroups(B * H * Nq, d) >= (int64_t(1) << 31))
    return fail(FA_ERR_SHAPE, "too many workgroups");
  iofa::FwdArgs a{Q, K, V, O, LSE, B * H, Nq, Nk, d, scale, dtype,
                  static_cast<hipStream_t>(stream)};
  if (g == 1) return hip_status(iofa::launch_fused(a), "fused forward launch");
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = o_part + static_cast<size_t>(g) * B * H * Nq * d;
  st = hip_status(iofa::launch_fused_partial(a, g, o_part, lse_part), "split-KV partial launch");
  if (st != FA_OK) return st;
  iofa::MergeArgs m{o_part, lse_part, g, B * H * Nq, d, O, LSE, dtype,
                    static_cast<hipStream_t>(stream)};
  return hip_status(iofa::launch_merge(m), "split-KV merge launch");
}

int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   void* workspace, size_t workspace_bytes, int num_splits, int64_t B, int64_t H,
                   int64_t N, int64_t d, float scale, int dtype, void* stream) {
  return fa_fwd_splitkv_qk(Q, K, V, O, LSE, workspace, workspace_bytes, num_splits, B, H, N, N,
                           d, scale, dtype, stream);
}

static_assert(FA_NOALLOC_SCRATCH_BYTES == iofa::kScratchBytes,
              "the header and the library state one scratch size");

int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int num_splits, int64_t B, int64_t H, int64_t N, int64_t d,
                           float scale, int dtype, void* stream) {
  g_last_error.clear();
  bool empty = false;
  int st = check_common(Q, K, V, O, LSE, true, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const size_t need = fa_splitkv_workspace_bytes(B, H, N, d, dtype, num_splits);
  if (need > FA_NOALLOC_SCRATCH_BYTES)
    return fail(FA_ERR_SHAPE, "the " + std::to_string(fa_splitkv_num_splits(B, H, N, d, dtype,
                                                                            num_splits)) +
                                  "-way split needs " + std::to_string(need) +
                                  " bytes of partials, more than the " +
                                  std::to_string(FA_NOALLOC_SCRATCH_BYTES) +
                                  "-byte scratch array: request fewer splits (1 needs none) "
                                  "or call fa_fwd_splitkv with a workspace");
  void* scratch = nullptr;
  if (need > 0) {
    st = hip_status(iofa::scratch_address(&scratch), "scratch array address");
    if (st != FA_OK) return st;
  }
  return fa_fwd_splitkv(Q, K, V, O, LSE, scratch, need, num_splits, B, H, N, d, scale, dtype,
                        stream);
}

int fa_merge_partials(const float* O_part, const float* LSE_part, int num_parts, int64_t rows,
                      int64_t d, void* O, float* LSE, int dtype, void* stream) {
  g_last_error.clear();
  if (elem_bytes(dtype) == 0)
    return fail(FA_ERR_DTYPE, "dtype " + std::to_string(dtype) + " is not FA_F32, FA_F16 or FA_BF16");
  if (num_parts < 1 || num_parts > kMaxMergeParts)
    return fail(FA_ERR_SHAPE, "num_parts must be in 1.." + std::to_string(kMaxMergeParts));
  if (rows < 0) return fail(FA_ERR_SHAPE, "rows must be >= 0");
  if (d != 64 && d != 128)
    return fail(FA_ERR_HEAD_DIM, "head dimension d must be 64 or 128 (got " + std::to_string(d) + ")");
  if (rows == 0) return FA_OK;
  if (rows > ((int64_t(1) << 40) - 1) / (num_parts * (d + 1)))
    return fail(FA_ERR_SHAPE, "too many rows");
  if (!O_part || !LSE_part || !O || !LSE) return fail(FA_ERR_NULL, "pointers must not be NULL");
  if (!aligned(O_part, 16) || !aligned(O, 16)) return fail(FA_ERR_ALIGN, "O_part and O must be 16-byte aligned");
  if (!aligned(LSE_part, 4) || !aligned(LSE, 4)) return fail(FA_ERR_ALIGN, "LSE_part and LSE must be 4-byte aligned");
  const size_t np = static_cast<size_t>(num_parts), r = static_cast<size_t>(rows);
  const Region in[2] = {{O_part, np * r * d * sizeof(float), "O_part"},
                        {LSE_part, np * r * sizeof(float), "LSE_part"}};
  const Region out[2] = {{O, r * d * elem_bytes(dtype), "O"}, {LSE, r * sizeof(float), "LSE"}};
  int st = check_aliasing(in, 2, out, 2);
  if (st != FA_OK) return st;
  if (iofa::merge_workgroups(rows, d) >= (int64_t(1) << 31))
    return fail(FA_ERR_SHAPE, "too many workgroups");
  iofa::MergeArgs m{O_part, LSE_part, num_parts, rows, d, O, LSE, dtype,
                    static_cast<hipStream_t>(stream)};
  return hip_status(iofa::launch_merge(m), "merge launch");
}

int fa_naive_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, void* S_ws,
                 void* P_ws, int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype,
                 void* stream) {
  g_last_error.clear();
  bool empty = false;
  int st = check_common(Q, K, V, O, LSE, false, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  if (!S_ws || !P_ws) return fail(FA_ERR_NULL, "S_ws and P_ws must not be NULL");
  if (!aligned(S_ws, 16) || !aligned(P_ws, 16))
    return fail(FA_ERR_ALIGN, "S_ws and P_ws must be 16-byte aligned");
  if (N > iofa::kNaiveMaxN)
    return fail(FA_ERR_SHAPE, "the naive path supports N <= " + std::to_string(iofa::kNaiveMaxN));
  const size_t tensor = static_cast<size_t>(B * H * N * d) * elem_bytes(dtype);
  const size_t lse = LSE ? static_cast<size_t>(B * H * N) * sizeof(float) : 0;
  const size_t ws = fa_naive_workspace_bytes(B, H, N, dtype);
  const Region in[3] = {{Q, tensor, "Q"}, {K, tensor, "K"}, {V, tensor, "V"}};
  const Region out[4] = {{O, tensor, "O"}, {LSE, lse, "LSE"}, {S_ws, ws, "S_ws"}, {P_ws, ws, "P_ws"}};
  st = check_aliasing(in, 3, out, 4);
  if (st != FA_OK) return st;
  if (iofa::naive_max_workgroups(dtype, B * H, N) >= (int64_t(1) << 31))
    return fail(FA_ERR_SHAPE, "too many workgroups");
  iofa::NaiveArgs a{{Q, K, V, O, LSE, B * H, N, N, d, scale, dtype, static_cast<hipStream_t>(stream)},
                    S_ws, P_ws, round_up8(N)};
  return hip_status(iofa::launch_naive(a), "naive forward launch");
}

size_t fa_softmax_workspace_bytes(int64_t rows, int64_t n, int dtype) {
  if (elem_bytes(dtype) == 0 || rows < 0 || n < 0) return 0;
  const int64_t chunk = iofa::softmax_chunk(dtype);
  if (n <= chunk) return 0;
  // two passes: a pair per chunk, then one per row
  const size_t two = product_or_zero({static_cast<size_t>(rows), static_cast<size_t>(ceil_div(n, chunk)) + 1,
                                      2 * sizeof(float)});
  // one pass: two counters, then a pair (8 bytes) and a flag (4) per slice
  const size_t one = product_or_zero({static_cast<size_t>(rows),
                                      static_cast<size_t>(ceil_div(n, iofa::softmax_slice(dtype))), 12});
  if (two == 0 || one == 0 || one > SIZE_MAX - 16) return 0;
  return std::max(two, one + 16);
}

int fa_softmax_rows(const void* X, void* Y, float* LSE, int64_t rows, int64_t n, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const int e = elem_bytes(dtype);
  if (e == 0)
    return fail(FA_ERR_DTYPE, "dtype " + std::to_string(dtype) + " is not FA_F32, FA_F16 or FA_BF16");
  if (rows < 0 || n < 0) return fail(FA_ERR_SHAPE, "rows and n must be >= 0");
  if (rows == 0 || n == 0) return FA_OK;
  const int64_t chunk = iofa::softmax_chunk(dtype);
  const int64_t pieces = ceil_div(n, iofa::softmax_piece(dtype));   // the largest grid per row
  if (pieces > INT32_MAX || rows > INT32_MAX / pieces)   // rows * pieces < 2^31
    return fail(FA_ERR_SHAPE, "too many workgroups");
  if (!X || !Y) return fail(FA_ERR_NULL, "X and Y must not be NULL");
  if (!aligned(X, e) || !aligned(Y, e)) return fail(FA_ERR_ALIGN, "X and Y must be element-aligned");
  if (LSE && !aligned(LSE, 4)) return fail(FA_ERR_ALIGN, "LSE must be 4-byte aligned");
  const size_t need = fa_softmax_workspace_bytes(rows, n, dtype);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_NULL, "workspace must not be NULL for rows longer than " +
                                                 std::to_string(chunk));
    if (!aligned(workspace, 8)) return fail(FA_ERR_ALIGN, "workspace must be 8-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_SHAPE, "workspace holds " + std::to_string(workspace_bytes) +
                                    " bytes, rows of this length need " + std::to_string(need));
  }
  // Y == X (in place) is allowed: every workgroup reads its piece in full
  // before writing it, and pass 2 starts after pass 1.  Partial overlap is not.
  const size_t bytes = static_cast<size_t>(rows) * static_cast<size_t>(n) * e;
  const Region in[1] = {{X, Y == X ? 0 : bytes, "X"}};
  const Region out[3] = {{Y, bytes, "Y"}, {LSE, LSE ? static_cast<size_t>(rows) * 4 : 0, "LSE"},
                         {workspace, need, "workspace"}};
  int st = check_aliasing(in, 1, out, 3);
  if (st == FA_OK && Y == X) {
    const Region xin[1] = {{X, bytes, "X"}};
    st = check_aliasing(xin, 1, out + 1, 2);
  }
  if (st != FA_OK) return st;
  iofa::SoftmaxArgs a{X, Y, LSE, rows, n, dtype, workspace, static_cast<hipStream_t>(stream)};
  return hip_status(iofa::launch_softmax(a), "softmax launch");
}

int fa_softmax_x_reads(const void* X, const void* Y, int64_t rows, int64_t n, int dtype) {
  if (elem_bytes(dtype) == 0 || rows <= 0 || n <= 0) return 0;
  const iofa::SoftmaxArgs a{X, const_cast<void*>(Y), nullptr, rows, n, dtype, nullptr, nullptr};
  return iofa::softmax_x_reads(a);
}

int fa_softmax_set_wait_limit(int polls) { return iofa::softmax_wait_limit(polls); }

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  return product_or_zero({static_cast<size_t>(B), static_cast<size_t>(H), static_cast<size_t>(N),
                          2 * sizeof(float)});
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
           int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype, void* stream) {
  g_last_error.clear();
  if (dtype == FA_F32) return fail(FA_ERR_DTYPE, "the backward pass takes FA_F16 or FA_BF16 inputs");
  bool empty = false;
  int st = check_common(Q, K, V, dQ, LSE, true, B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  if (!O || !dO || !dK || !dV) return fail(FA_ERR_NULL, "O, dO, dK and dV must not be NULL");
  if (!aligned(O, 16) || !aligned(dO, 16) || !aligned(dK, 16) || !aligned(dV, 16))
    return fail(FA_ERR_ALIGN, "O, dO, dK and dV must be 16-byte aligned");
  const size_t need = fa_bwd_workspace_bytes(B, H, N);
  if (!workspace) return fail(FA_ERR_NULL, "workspace must not be NULL");
  if (!aligned(workspace, 16)) return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_SHAPE, "workspace holds " + std::to_string(workspace_bytes) +
                                  " bytes, the backward pass needs " + std::to_string(need));
  const size_t tensor = static_cast<size_t>(B * H * N * d) * elem_bytes(dtype);
  const size_t lse = static_cast<size_t>(B * H * N) * sizeof(float);
  const Region in[6] = {{Q, tensor, "Q"}, {K, tensor, "K"}, {V, tensor, "V"},
                        {O, tensor, "O"}, {dO, tensor, "dO"}, {LSE, lse, "LSE"}};
  const Region out[4] = {{dQ, tensor, "dQ"}, {dK, tensor, "dK"}, {dV, tensor, "dV"},
                         {workspace, need, "workspace"}};
  st = check_aliasing(in, 6, out, 4);
  if (st != FA_OK) return st;
  if (iofa::bwd_workgroups(B * H, N) >= (int64_t(1) << 31))
    return fail(FA_ERR_SHAPE, "too many workgroups");
  iofa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B * H, N, d, scale, dtype,
                  static_cast<hipStream_t>(stream)};
  return hip_status(iofa::launch_bwd(a), "backward launch");
}

size_t fa_naive_workspace_bytes(int64_t B, int64_t H, int64_t N, int dtype) {
  const int e = elem_bytes(dtype);
  if (e == 0 || B < 0 || H < 0 || N < 0 || N > iofa::kNaiveMaxN) return 0;
  return product_or_zero({static_cast<size_t>(B), static_cast<size_t>(H), static_cast<size_t>(N),
                          static_cast<size_t>(round_up8(N)), static_cast<size_t>(e)});
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "invalid shape";
    case FA_ERR_HEAD_DIM: return "unsupported head dimension";
    case FA_ERR_DTYPE: return "unsupported dtype";
    case FA_ERR_ALIGN: return "misaligned pointer";
    case FA_ERR_SCALE: return "non-finite scale";
    case FA_ERR_ALIAS: return "overlapping buffers";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return 400; }

}  // extern "C"
