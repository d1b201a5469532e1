// Internal interface between the C ABI (fa_api.cpp) and the kernel files.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int64_t N;
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

// Workgroups the fused launch uses (for the grid-size limit check).
int64_t fused_workgroups(int dtype, int64_t BH, int64_t N);
// Largest grid among the naive path's three launches.
int64_t naive_max_workgroups(int dtype, int64_t BH, int64_t N);

hipError_t launch_fused(const FwdArgs& a);
hipError_t launch_naive(const NaiveArgs& a);

constexpr int64_t kNaiveMaxN = 32768;

}  // namespace iofa
