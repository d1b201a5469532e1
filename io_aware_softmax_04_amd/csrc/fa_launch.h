// Internal interface between the C ABI (fa_api.cpp) and the kernel files.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace iofa {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeF16 = 1;
constexpr int kDtypeBF16 = 2;

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int64_t BH;  // B * H
  int64_t N;   // query rows per head (Q, O, LSE)
  int64_t Nk;  // key rows per head (K, V): N itself for self-attention
  int64_t d;
  float scale;
  int dtype;
  hipStream_t stream;
};

struct NaiveArgs {
  FwdArgs f;
  void* S;
  void* P;
  int64_t ldS;  // row stride of S and P in elements (N rounded up to 8)
};

// Merge of G fp32 partials (G, rows, d) / (G, rows) into O (rows, d) in
// `dtype` and LSE (rows).
struct MergeArgs {
  const float* O_part;
  const float* LSE_part;
  int G;
  int64_t rows;
  int64_t d;
  void* O;
  float* LSE;
  int dtype;
  hipStream_t stream;
};

// Row softmax of X (rows, n) into Y.  Workspace for rows longer than one
// chunk: the two-pass form uses rows * (chunks + 1) float2 (m, l) pairs, the
// resident form 16 + 12 * rows * parts bytes (parts = slices per row).
struct SoftmaxArgs {
  const void* X;
  void* Y;
  float* LSE;   // may be NULL
  int64_t rows;
  int64_t n;
  int dtype;
  void* workspace;
  hipStream_t stream;
};
// Elements of a row one workgroup covers in the one-chunk form and in pass 1.
int64_t softmax_chunk(int dtype);
// Elements of one slice (task) of the resident form.
int64_t softmax_slice(int dtype);
// Elements one workgroup of pass 2 covers on 16-byte-aligned rows (the
// smallest piece any launch uses).
int64_t softmax_piece(int dtype);
hipError_t launch_softmax(const SoftmaxArgs& a);
// How many times launch_softmax(a) reads X from memory (1 or 2).
int softmax_x_reads(const SoftmaxArgs& a);
// Sets the resident form's bound on each wait (polls; negative restores the
// default) and returns the previous bound.
int softmax_wait_limit(int polls);

// Backward pass (16-bit inputs): dQ, dK, dV from Q, K, V, O, dO and the
// forward's LSE; stats: B*H*N float2 workspace of (LSE * log2 e, D).
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  void* dQ;
  void* dK;
  void* dV;
  void* stats;
  int64_t BH;
  int64_t N;
  int64_t d;
  float scale;
  int dtype;
  hipStream_t stream;
};
int64_t bwd_workgroups(int64_t BH, int64_t N);
hipError_t launch_bwd(const BwdArgs& a);

// FP8 (E4M3) forward: Q, K, V codes (B*H, N, d), O bf16, LSE fp32.
struct Fp8Args {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int64_t BH;
  int64_t N;
  int64_t d;
  float c2;        // |scale| * q_scale * k_scale * log2(e)
  float v_scale;
  bool negate_q;   // scale < 0: Q's signs are flipped on load
  hipStream_t stream;
};
int64_t fp8_workgroups(int64_t BH, int64_t N);
hipError_t launch_fp8(const Fp8Args& a);

// Keys per tile of the fused kernels, and query rows per workgroup of their
// form with the most workgroups.
int fused_key_tile(int dtype, int64_t d);
int64_t fused_query_tile(int dtype);
// At most this many workgroups per fused launch (the grid-size limit check).
int64_t fused_workgroups(int dtype, int64_t BH, int64_t N, int64_t splits);
// Waves of a fused launch (the split-KV heuristic).
int64_t fused_waves(int dtype, int64_t BH, int64_t N, int64_t splits);
int64_t merge_workgroups(int64_t rows, int64_t d);
// Largest grid among the naive path's three launches.
int64_t naive_max_workgroups(int dtype, int64_t BH, int64_t N);

hipError_t launch_fused(const FwdArgs& a);
// Partial pass of the split-KV forward: fp32 O_part (splits, B*H, N, d) and
// LSE_part (splits, B*H, N).
hipError_t launch_fused_partial(const FwdArgs& a, int splits, float* O_part, float* LSE_part);
hipError_t launch_merge(const MergeArgs& a);
hipError_t launch_naive(const NaiveArgs& a);

constexpr int64_t kNaiveMaxN = 32768;

// Bytes of the library's own scratch array (fa_scratch_gfx950.hip), used by
// the entry point that allocates nothing; FA_NOALLOC_SCRATCH_BYTES in
// fa_api.h states the same size.
constexpr size_t kScratchBytes = size_t(64) << 20;
// Device address of the current device's copy of that array (looked up once
// per device, then cached).
hipError_t scratch_address(void** ptr);

}  // namespace iofa
