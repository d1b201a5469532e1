// Row-wise softmax y = e^{x - m} / l for (rows, n) matrices, gfx950.
//
// The online-softmax idea of xinc.fun archive 235, "7. Online Softmax"
// (keep only a running maximum m and denominator l; a new block of values
// rescales the old l by e^{m_old - m_new}), used as its own memory-bound
// operation: a row is cut into chunks of one workgroup's size; each chunk
// yields its own (m, l), and the chunks' pairs combine with the block merge
// of the special-jiahao.github.io "Flash Attention" note, section
// "增量求解 softmax" (m = max(m1, m2), l = l1 e^{m1-m} + l2 e^{m2-m}).
//
//   rows that fit one chunk:  one kernel; the chunk stays in registers, so x
//                             is read once and y written once;
//   longer rows:              pass 1 writes every chunk's (m, l) (x read
//                             once), pass 2 merges the row's pairs and
//                             writes its chunk of y (x read again); one
//                             workgroup per (row, chunk), flattened.
// The naive three-pass form (maximum, sum, normalise) reads x three times.
//
// Workgroup = 256 threads; a thread holds EPT elements loaded as 16-byte
// vectors when a row's length keeps rows 16-byte aligned (VEC elements per
// load), else one element per load.  Arithmetic is fp32.  fp32 outputs use
// the accurate expf; 16-bit outputs use the hardware exp2 (see exp_nonpos),
// whose relative error (below 2e-5 while the result is above bf16's
// smallest subnormal) is far under the output's own rounding and which costs
// three instructions instead of about twelve, so the kernels stay bound by
// memory rather than by the vector unit.
#include "fa_device.h"
#include "fa_launch.h"

namespace iofa {

namespace {

constexpr int kThreads = 256;

template <int KIND>   // 0: fp32, 1: fp16, 2: bf16
struct Elem {
  static constexpr int BYTES = KIND == 0 ? 4 : 2;
  static constexpr int VEC = 16 / BYTES;             // elements per 16-byte load
  static constexpr int EPT = KIND == 0 ? 16 : 32;    // elements per thread
  static constexpr int CHUNK = kThreads * EPT;       // elements per workgroup
  __device__ static inline float load1(const void* p, int64_t i) {
    if constexpr (KIND == 0) return static_cast<const float*>(p)[i];
    const uint16_t b = static_cast<const uint16_t*>(p)[i];
    if constexpr (KIND == 2) return __uint_as_float(static_cast<uint32_t>(b) << 16);
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
  __device__ static inline void store1(void* p, int64_t i, float v) {
    if constexpr (KIND == 0) static_cast<float*>(p)[i] = v;
    else if constexpr (KIND == 2) static_cast<uint16_t*>(p)[i] = Bf16::bits(v);
    else static_cast<uint16_t*>(p)[i] = F16::bits(v);
  }
  // VEC consecutive elements at element index i (16-byte aligned)
  __device__ static inline void loadv(const void* p, int64_t i, float* v) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p) + i * BYTES);
    if constexpr (KIND == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = half_of(w, e);
        v[e] = KIND == 2 ? __uint_as_float(h << 16)
                         : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
      }
    }
  }
  __device__ static inline void storev(void* p, int64_t i, const float* v) {
    u32x4 w;
    if constexpr (KIND == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = KIND == 2 ? Bf16::pack(v[2 * e], v[2 * e + 1]) : F16::pack(v[2 * e], v[2 * e + 1]);
    }
    *reinterpret_cast<u32x4*>(static_cast<char*>(p) + i * BYTES) = w;
  }
};

// 2^bias * e^t for t <= 0 (t = x - m): the accurate expf (bias 0) for fp32
// outputs, the hardware exp2 of t log2 e + 64 for 16-bit ones.  v_exp_f32
// flushes subnormal results; the bias keeps every result above e^-133 (the
// smallest bf16 subnormal is 2^-133) in fp32's normal range.  The same factor
// scales every l, so the block merge and y = (2^bias e^t) / l are unchanged
// and only the log-sum-exp subtracts it (row sums stay below 2^95).
template <int KIND>
constexpr float kExpBias = KIND == 0 ? 0.f : 64.f;
template <int KIND>
__device__ inline float exp_nonpos(float t) {
  if constexpr (KIND == 0) return expf(t);
  return __builtin_amdgcn_exp2f(fmaf(t, kLog2e, kExpBias<KIND>));
}
// ln l - bias ln 2: the log-sum-exp's share of the row sum.
template <int KIND>
__device__ inline float log_sum(float l) {
  return logf(l) - kExpBias<KIND> * kLn2;
}

// Block merge of two (m, l) pairs; -inf maxima (no values yet) merge as the
// identity.
__device__ inline float2 merge_ml(float2 a, float2 b) {
  const float m = fmaxf(a.x, b.x);
  if (m == -__builtin_inff()) return make_float2(m, 0.f);
  return make_float2(m, a.y * expf(a.x - m) + b.y * expf(b.x - m));
}

__device__ inline float2 wave_merge(float2 v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float2 o = make_float2(__shfl_xor(v.x, off, 64), __shfl_xor(v.y, off, 64));
    v = merge_ml(v, o);
  }
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Workgroup-wide reduction of one value per thread (4 waves).
template <class F>
__device__ inline float block_reduce(float v, float* red, F op) {
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return op(op(red[0], red[1]), op(red[2], red[3]));
}

// Loads the chunk [c0, c0 + CHUNK) of one row (length n) into v; elements
// past the row are -inf.  Thread t holds, for load step i, the VEC
// elements at c0 + (i * 256 + t) * VEC (coalesced).
template <int KIND, bool VECTOR>
__device__ inline void load_chunk(const void* row, int64_t n, int64_t c0, float* v) {
  using E = Elem<KIND>;
  constexpr int W = VECTOR ? E::VEC : 1;
#pragma unroll
  for (int i = 0; i < E::EPT / W; ++i) {
    const int64_t e0 = c0 + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * W;
    if (VECTOR && e0 + W <= n) {
      E::loadv(row, e0, v + i * W);
    } else {
#pragma unroll
      for (int e = 0; e < W; ++e) v[i * W + e] = (e0 + e < n) ? E::load1(row, e0 + e) : -__builtin_inff();
    }
  }
}

template <int KIND, bool VECTOR>
__device__ inline void store_chunk(void* row, int64_t n, int64_t c0, const float* v) {
  using E = Elem<KIND>;
  constexpr int W = VECTOR ? E::VEC : 1;
#pragma unroll
  for (int i = 0; i < E::EPT / W; ++i) {
    const int64_t e0 = c0 + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * W;
    if (VECTOR && e0 + W <= n) {
      E::storev(row, e0, v + i * W);
    } else {
#pragma unroll
      for (int e = 0; e < W; ++e)
        if (e0 + e < n) E::store1(row, e0 + e, v[i * W + e]);
    }
  }
}

// (m, l) of the values in v (some may be -inf).
template <int KIND, int EPT>
__device__ inline float2 chunk_stats(const float* v, float* red) {
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, v[i]);
  m = block_reduce(wave_max(m), red, [](float a, float b) { return fmaxf(a, b); });
  if (m == -__builtin_inff()) return make_float2(m, 0.f);
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) l += exp_nonpos<KIND>(v[i] - m);
  l = block_reduce(wave_sum(l), red, [](float a, float b) { return a + b; });
  return make_float2(m, l);
}

// Rows of at most one chunk: read once, write once.  X and Y may be the same
// buffer (an in-place call), so neither is declared __restrict__: each thread
// reads its elements before it writes them, and no other thread touches them.
template <int KIND, bool VECTOR>
__global__ __launch_bounds__(kThreads) void softmax_short_kernel(const void* X, void* Y,
                                                                 float* __restrict__ LSE,
                                                                 int64_t n) {
  using E = Elem<KIND>;
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const char* xr = static_cast<const char*>(X) + r * n * E::BYTES;
  char* yr = static_cast<char*>(Y) + r * n * E::BYTES;
  float v[E::EPT];
  load_chunk<KIND, VECTOR>(xr, n, 0, v);
  const float2 ml = chunk_stats<KIND, E::EPT>(v, red);
  const float inv = 1.f / ml.y;
#pragma unroll
  for (int i = 0; i < E::EPT; ++i) v[i] = exp_nonpos<KIND>(v[i] - ml.x) * inv;
  store_chunk<KIND, VECTOR>(yr, n, 0, v);
  if (LSE && threadIdx.x == 0) LSE[r] = ml.x + log_sum<KIND>(ml.y);
}

// Long rows, pass 1: (m, l) of chunk c of row r (workgroup r * chunks + c).
template <int KIND, bool VECTOR>
__global__ __launch_bounds__(kThreads) void softmax_stats_kernel(const void* __restrict__ X,
                                                                 float2* __restrict__ stats,
                                                                 int64_t n, int chunks) {
  using E = Elem<KIND>;
  __shared__ float red[4];
  const int64_t r = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const char* xr = static_cast<const char*>(X) + r * n * E::BYTES;
  float v[E::EPT];
  load_chunk<KIND, VECTOR>(xr, n, c * E::CHUNK, v);
  const float2 ml = chunk_stats<KIND, E::EPT>(v, red);
  if (threadIdx.x == 0) stats[r * chunks + c] = ml;
}

// Long rows, pass 2: merge row r's chunk pairs, write its chunk c.  X and Y
// may be the same buffer (in place), as in softmax_short_kernel.
template <int KIND, bool VECTOR>
__global__ __launch_bounds__(kThreads) void softmax_normalize_kernel(
    const void* X, void* Y, float* __restrict__ LSE,
    const float2* __restrict__ stats, int64_t n, int chunks) {
  using E = Elem<KIND>;
  __shared__ float2 red2[4];
  const int64_t r = blockIdx.x / chunks, c = blockIdx.x % chunks;
  float2 ml = make_float2(-__builtin_inff(), 0.f);
  for (int i = threadIdx.x; i < chunks; i += kThreads) ml = merge_ml(ml, stats[r * chunks + i]);
  ml = wave_merge(ml);
  if ((threadIdx.x & 63) == 0) red2[threadIdx.x >> 6] = ml;
  __syncthreads();
  ml = merge_ml(merge_ml(red2[0], red2[1]), merge_ml(red2[2], red2[3]));
  const char* xr = static_cast<const char*>(X) + r * n * E::BYTES;
  char* yr = static_cast<char*>(Y) + r * n * E::BYTES;
  float v[E::EPT];
  load_chunk<KIND, VECTOR>(xr, n, c * E::CHUNK, v);
  const float inv = 1.f / ml.y;
#pragma unroll
  for (int i = 0; i < E::EPT; ++i) v[i] = exp_nonpos<KIND>(v[i] - ml.x) * inv;
  store_chunk<KIND, VECTOR>(yr, n, c * E::CHUNK, v);
  if (LSE && c == 0 && threadIdx.x == 0) LSE[r] = ml.x + log_sum<KIND>(ml.y);
}

template <int KIND, bool VECTOR>
hipError_t launch_softmax_t(const SoftmaxArgs& a) {
  using E = Elem<KIND>;
  if (a.n <= E::CHUNK) {
    hipLaunchKernelGGL((softmax_short_kernel<KIND, VECTOR>), dim3(static_cast<unsigned>(a.rows)),
                       dim3(kThreads), 0, a.stream, a.X, a.Y, a.LSE, a.n);
    return hipGetLastError();
  }
  const int chunks = static_cast<int>((a.n + E::CHUNK - 1) / E::CHUNK);
  const unsigned wg = static_cast<unsigned>(a.rows * chunks);
  float2* stats = static_cast<float2*>(a.workspace);
  hipLaunchKernelGGL((softmax_stats_kernel<KIND, VECTOR>), dim3(wg), dim3(kThreads), 0, a.stream,
                     a.X, stats, a.n, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_normalize_kernel<KIND, VECTOR>), dim3(wg), dim3(kThreads), 0,
                     a.stream, a.X, a.Y, a.LSE, stats, a.n, chunks);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_softmax_k(const SoftmaxArgs& a) {
  using E = Elem<KIND>;
  const bool vec = (a.n % E::VEC) == 0 && (reinterpret_cast<uintptr_t>(a.X) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.Y) % 16) == 0;
  return vec ? launch_softmax_t<KIND, true>(a) : launch_softmax_t<KIND, false>(a);
}

}  // namespace

int64_t softmax_chunk(int dtype) { return dtype == kDtypeF32 ? Elem<0>::CHUNK : Elem<2>::CHUNK; }

hipError_t launch_softmax(const SoftmaxArgs& a) {
  if (a.dtype == kDtypeBF16) return launch_softmax_k<2>(a);
  if (a.dtype == kDtypeF16) return launch_softmax_k<1>(a);
  return launch_softmax_k<0>(a);
}

}  // namespace iofa
