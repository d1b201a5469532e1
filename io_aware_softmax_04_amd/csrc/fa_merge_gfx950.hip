// Merge of partial attention results over disjoint key ranges (gfx950).
//
// The special-jiahao.github.io "Flash Attention" note, section
// "增量求解 softmax", combines the local softmaxes of two blocks of a vector
// into the global one: the global maximum, each block's denominator rescaled
// by e^{m(block) - m(x)}, and each block's local result weighted by its
// rescaled denominator over the global one.  For G blocks of keys with
// partial outputs O_g (each normalised by its own denominator) and
// log-sum-exps LSE_g = m_g + ln l_g this reads, per query row,
//     LSE = ln sum_g e^{LSE_g},      O = sum_g e^{LSE_g - LSE} O_g,
// since e^{LSE_g - LSE} = l(block g)^global / l(x).
//
// Memory-bound: each row reads G*(d + 1) fp32 values and writes d outputs
// and one LSE.  A row is handled by d/4 threads, each owning 4 consecutive
// columns (16-byte loads); a 256-thread workgroup covers 256/(d/4) rows.
// The largest LSE_g is the reference, so no exponential exceeds 1; exp and
// log are the accurate library functions (the kernel is bandwidth-bound).
#include "fa_device.h"
#include "fa_launch.h"

namespace iofa {

namespace {

template <int KIND>   // 0: fp32 output, 1: fp16, 2: bf16
__device__ inline void store4(void* O, size_t off, float4 v) {
  if constexpr (KIND == 0) {
    *reinterpret_cast<float4*>(static_cast<float*>(O) + off) = v;
  } else {
    using T = typename std::conditional<KIND == 2, Bf16, F16>::type;
    u32x2 w;
    w[0] = T::pack(v.x, v.y);
    w[1] = T::pack(v.z, v.w);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(O) + off) = w;
  }
}

template <int KIND, int D, int U>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ Op,
                                                       const float* __restrict__ Lp, int G,
                                                       int64_t rows, void* __restrict__ O,
                                                       float* __restrict__ LSE) {
  constexpr int TPR = D / 4;           // threads per row
  constexpr int RPB = 256 / TPR;       // rows per workgroup
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  if (row >= rows) return;

  // Loads are issued in groups of U partials (the smallest power of two
  // covering G, 16 for G > 8) before any of them is used, so a call with few
  // rows (one decode row per head) waits for one memory round trip per group
  // instead of one per partial; the arithmetic runs in partial order either
  // way.  Slots past the last partial load partial G - 1 again (no branch
  // around a load) and are left out of the sums.  The first group's values
  // stay in registers between the two passes; past it the maximum reads the
  // LSEs LC at a time.
  float lp[U];
  float4 op[U];
  auto load_group = [&](int g0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t g = g0 + u < G ? g0 + u : G - 1;
      lp[u] = Lp[g * rows + row];
      op[u] = *reinterpret_cast<const float4*>(Op + (g * rows + row) * D + 4 * c4);
    }
  };
  load_group(0);
  float ref = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < U; ++u) ref = fmaxf(ref, lp[u]);
  constexpr int LC = U > 8 ? 32 : U;
  for (int g0 = U; g0 < G; g0 += LC) {
    float l[LC];
#pragma unroll
    for (int u = 0; u < LC; ++u) l[u] = Lp[static_cast<int64_t>(g0 + u < G ? g0 + u : G - 1) * rows + row];
#pragma unroll
    for (int u = 0; u < LC; ++u) ref = fmaxf(ref, l[u]);
  }
  const float base = (ref == -__builtin_inff()) ? 0.f : ref;
  float total = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float lse_g, float4 o) {
    const float w = expf(lse_g - base);
    total += w;
    acc.x = fmaf(w, o.x, acc.x);
    acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z);
    acc.w = fmaf(w, o.w, acc.w);
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < G) add(lp[u], op[u]);
  for (int g0 = U; g0 < G; g0 += U) {
    load_group(g0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (g0 + u < G) add(lp[u], op[u]);
  }
  // total >= 1 whenever some block has keys (the reference block weighs 1)
  const float inv = total > 0.f ? 1.f / total : 0.f;
  store4<KIND>(O, static_cast<size_t>(row) * D + 4 * c4,
               make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
  if (c4 == 0) LSE[row] = total > 0.f ? base + logf(total) : -__builtin_inff();
}

template <int KIND, int D, int U>
hipError_t launch_merge_u(const MergeArgs& a) {
  constexpr int RPB = 256 / (D / 4);
  const int64_t wg = (a.rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((fa_merge_kernel<KIND, D, U>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                     a.stream, a.O_part, a.LSE_part, a.G, a.rows, a.O, a.LSE);
  return hipGetLastError();
}

template <int KIND, int D>
hipError_t launch_merge_t(const MergeArgs& a) {
  if (a.G <= 1) return launch_merge_u<KIND, D, 1>(a);
  if (a.G == 2) return launch_merge_u<KIND, D, 2>(a);
  if (a.G <= 4) return launch_merge_u<KIND, D, 4>(a);
  if (a.G <= 8) return launch_merge_u<KIND, D, 8>(a);
  return launch_merge_u<KIND, D, 16>(a);
}

}  // namespace

int64_t merge_workgroups(int64_t rows, int64_t d) {
  const int64_t rpb = 256 / (d / 4);
  return (rows + rpb - 1) / rpb;
}

hipError_t launch_merge(const MergeArgs& a) {
  if (a.d == 128) {
    if (a.dtype == kDtypeBF16) return launch_merge_t<2, 128>(a);
    if (a.dtype == kDtypeF16) return launch_merge_t<1, 128>(a);
    return launch_merge_t<0, 128>(a);
  }
  if (a.dtype == kDtypeBF16) return launch_merge_t<2, 64>(a);
  if (a.dtype == kDtypeF16) return launch_merge_t<1, 64>(a);
  return launch_merge_t<0, 64>(a);
}

}  // namespace iofa
