// Row-wise softmax y = e^{x - m} / l for (rows, n) matrices, gfx950.
//
// The online-softmax idea of xinc.fun archive 235, "7. Online Softmax"
// (keep only a running maximum m and denominator l; a new block of values
// rescales the old l by e^{m_old - m_new}), used as its own memory-bound
// operation: a row is cut into pieces, each piece yields its own (m, l), and
// the pieces' pairs combine with the block merge of the special-jiahao.github.io
// "Flash Attention" note, section "增量求解 softmax"
// (m = max(m1, m2), l = l1 e^{m1-m} + l2 e^{m2-m}).  Three forms:
//
//   rows of one chunk:   one workgroup per row holds the row in registers;
//                        x is read once and y written once;
//   resident rows:       rows of at most kResidentParts slices of 16384
//                        (16-bit) or 8192 (fp32) elements, 16-byte aligned:
//                        one workgroup per slice holds it in registers,
//                        publishes its pair, waits for the row's other
//                        slices and writes y from the registers (x read
//                        once; see the resident section below);
//   longer rows:         pass 1 writes every chunk's (m, l), a small kernel
//                        merges each row's pairs into one, pass 2 writes y
//                        (x read twice).
// The naive three-pass form (maximum, sum, normalise) reads x three times.
//
// Workgroup = 256 threads; a thread holds its elements as 16-byte vectors
// when the row length keeps rows 16-byte aligned (VEC elements per load),
// else one element per load.  Every access to x and y is non-temporal: each
// element is touched once per pass, so nothing is worth keeping in the
// caches.  Arithmetic is fp32.  fp32 outputs use the accurate expf; 16-bit
// outputs use the hardware exp2 (see exp_nonpos), whose relative error
// (below 2e-5 while the result is above bf16's smallest subnormal) is far
// under the output's own rounding and which costs three instructions instead
// of about twelve, so the kernels stay bound by memory rather than by the
// vector unit.
#include "fa_device.h"
#include "fa_launch.h"

#include <algorithm>
#include <atomic>

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
  // The 16-byte word of VEC consecutive elements at element index i
  // (16-byte aligned), and its values.
  __device__ static inline u32x4 loadw(const void* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const char*>(p) + i * BYTES));
  }
  __device__ static inline void unpack(const u32x4& w, float* v) {
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
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<char*>(p) + i * BYTES));
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

// Workgroup-wide (m, l) of one pair per wave (4 waves): every thread gets
// the merged pair.  red2 must not be in use by another step.
__device__ inline float2 merge_waves(float2 wave_pair, float2* red2) {
  if ((threadIdx.x & 63) == 0) red2[threadIdx.x >> 6] = wave_pair;
  __syncthreads();
  return merge_ml(merge_ml(red2[0], red2[1]), merge_ml(red2[2], red2[3]));
}

// Workgroup-wide block merge of one pair per thread.
__device__ inline float2 block_merge(float2 ml, float2* red2) {
  return merge_waves(wave_merge(ml), red2);
}

// (m, l) of the EPT values a thread holds in v (some may be -inf), over the
// workgroup: the wave's maximum first, then every lane sums against it, so
// a wave needs one max and one sum reduction; the four waves' pairs merge.
template <int KIND, int EPT>
__device__ inline float2 block_pair(const float* v, float2* red2) {
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float l = 0.f;
  if (m != -__builtin_inff()) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) l += exp_nonpos<KIND>(v[i] - m);
  }
  return merge_waves(make_float2(m, wave_sum(l)), red2);
}

// Loads EPT elements per thread of the piece starting at element c0 of one
// row (length n) into v; elements past the row are -inf.  Thread t holds,
// for load step i, the W elements at c0 + (i * 256 + t) * W (coalesced),
// W = VEC for 16-byte vectors (n is then a multiple of VEC, so a vector lies
// wholly inside the row or wholly past it, and the loads have no per-element
// branch between them), else 1.
template <int KIND, bool VECTOR, int EPT = Elem<KIND>::EPT>
__device__ inline void load_chunk(const void* row, int64_t n, int64_t c0, float* v) {
  using E = Elem<KIND>;
  constexpr int W = VECTOR ? E::VEC : 1;
  if constexpr (VECTOR) {
    // All words first, with no branch between the loads so that they go out
    // back to back: a vector past the row loads the row's last vector
    // instead (n >= VEC) and its values are replaced by -inf below.
    u32x4 w[EPT / W];
#pragma unroll
    for (int i = 0; i < EPT / W; ++i) {
      const int64_t e0 = c0 + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * W;
      w[i] = E::loadw(row, e0 < n ? e0 : n - W);
    }
#pragma unroll
    for (int i = 0; i < EPT / W; ++i) {
      const int64_t e0 = c0 + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * W;
      if (e0 < n) {
        E::unpack(w[i], v + i * W);
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) v[i * W + e] = -__builtin_inff();
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int64_t e0 = c0 + static_cast<int64_t>(i) * kThreads + threadIdx.x;
      v[i] = e0 < n ? E::load1(row, e0) : -__builtin_inff();
    }
  }
}

template <int KIND, bool VECTOR, int EPT = Elem<KIND>::EPT>
__device__ inline void store_chunk(void* row, int64_t n, int64_t c0, const float* v) {
  using E = Elem<KIND>;
  constexpr int W = VECTOR ? E::VEC : 1;
#pragma unroll
  for (int i = 0; i < EPT / W; ++i) {
    const int64_t e0 = c0 + (static_cast<int64_t>(i) * kThreads + threadIdx.x) * W;
    if (e0 < n) {
      if constexpr (VECTOR) E::storev(row, e0, v + i * W);
      else E::store1(row, e0, v[i]);
    }
  }
}

// Rows of at most one chunk: read once, write once.  X and Y may be the same
// buffer (an in-place call), so neither is declared __restrict__: each thread
// reads its elements before it writes them, and no other thread touches them.
template <int KIND, bool VECTOR>
__global__ __launch_bounds__(kThreads) void softmax_short_kernel(const void* X, void* Y,
                                                                 float* __restrict__ LSE,
                                                                 int64_t n) {
  using E = Elem<KIND>;
  __shared__ float2 red2[4];
  const int64_t r = blockIdx.x;
  const char* xr = static_cast<const char*>(X) + r * n * E::BYTES;
  char* yr = static_cast<char*>(Y) + r * n * E::BYTES;
  float v[E::EPT];
  load_chunk<KIND, VECTOR>(xr, n, 0, v);
  const float2 ml = block_pair<KIND, E::EPT>(v, red2);
  const float inv = 1.f / ml.y;
#pragma unroll
  for (int i = 0; i < E::EPT; ++i) v[i] = exp_nonpos<KIND>(v[i] - ml.x) * inv;
  store_chunk<KIND, VECTOR>(yr, n, 0, v);
  if (LSE && threadIdx.x == 0) LSE[r] = ml.x + log_sum<KIND>(ml.y);
}

// ---- Longer rows, two passes ----

// Pass 1: (m, l) of chunk c of row r (workgroup r * chunks + c).
template <int KIND, bool VECTOR>
__global__ __launch_bounds__(kThreads) void softmax_stats_kernel(const void* __restrict__ X,
                                                                 float2* __restrict__ stats,
                                                                 int64_t n, int chunks) {
  using E = Elem<KIND>;
  __shared__ float2 red2[4];
  const int64_t r = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const char* xr = static_cast<const char*>(X) + r * n * E::BYTES;
  float v[E::EPT];
  load_chunk<KIND, VECTOR>(xr, n, c * E::CHUNK, v);
  const float2 ml = block_pair<KIND, E::EPT>(v, red2);
  if (threadIdx.x == 0) stats[r * chunks + c] = ml;
}

// Between the passes: merges row r's chunk pairs into rowstats[r] (and writes
// its log-sum-exp), so that pass 2 reads one pair per workgroup.
template <int KIND>
__global__ __launch_bounds__(kThreads) void softmax_rowmerge_kernel(const float2* __restrict__ stats,
                                                                    float2* __restrict__ rowstats,
                                                                    float* __restrict__ LSE,
                                                                    int chunks) {
  __shared__ float2 red2[4];
  const int64_t r = blockIdx.x;
  float2 ml = make_float2(-__builtin_inff(), 0.f);
  for (int i = threadIdx.x; i < chunks; i += kThreads) ml = merge_ml(ml, stats[r * chunks + i]);
  ml = block_merge(ml, red2);
  if (threadIdx.x == 0) {
    rowstats[r] = ml;
    if (LSE) LSE[r] = ml.x + log_sum<KIND>(ml.y);
  }
}

// Pass 2: writes piece c (EPT elements per thread) of row r with the row's
// merged pair.  X and Y may be the same buffer (in place), as in
// softmax_short_kernel; pass 1 has read all of X before pass 2 starts.
template <int KIND, bool VECTOR, int EPT>
__global__ __launch_bounds__(kThreads) void softmax_normalize_kernel(
    const void* X, void* Y, const float2* __restrict__ rowstats, int64_t n, int pieces) {
  using E = Elem<KIND>;
  constexpr int64_t PIECE = static_cast<int64_t>(kThreads) * EPT;
  const int64_t r = blockIdx.x / pieces, c = blockIdx.x % pieces;
  const char* xr = static_cast<const char*>(X) + r * n * E::BYTES;
  char* yr = static_cast<char*>(Y) + r * n * E::BYTES;
  float v[EPT];
  load_chunk<KIND, VECTOR, EPT>(xr, n, c * PIECE, v);
  const float2 ml = rowstats[r];
  const float inv = 1.f / ml.y;
#pragma unroll
  for (int i = 0; i < EPT; ++i) v[i] = exp_nonpos<KIND>(v[i] - ml.x) * inv;
  store_chunk<KIND, VECTOR, EPT>(yr, n, c * PIECE, v);
}

// Elements per thread in pass 2: one 16-byte vector on aligned rows (small
// workgroups stream best there), a whole chunk's share otherwise.
template <int KIND, bool VECTOR>
constexpr int kNormEpt = VECTOR ? Elem<KIND>::VEC : Elem<KIND>::EPT;

template <int KIND, bool VECTOR>
hipError_t launch_two_pass(const SoftmaxArgs& a) {
  using E = Elem<KIND>;
  constexpr int EPT2 = kNormEpt<KIND, VECTOR>;
  constexpr int64_t PIECE = static_cast<int64_t>(kThreads) * EPT2;
  const int chunks = static_cast<int>((a.n + E::CHUNK - 1) / E::CHUNK);
  const int pieces = static_cast<int>((a.n + PIECE - 1) / PIECE);
  float2* stats = static_cast<float2*>(a.workspace);
  float2* rowstats = stats + a.rows * chunks;
  hipLaunchKernelGGL((softmax_stats_kernel<KIND, VECTOR>), dim3(static_cast<unsigned>(a.rows * chunks)),
                     dim3(kThreads), 0, a.stream, a.X, stats, a.n, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_rowmerge_kernel<KIND>), dim3(static_cast<unsigned>(a.rows)), dim3(kThreads),
                     0, a.stream, stats, rowstats, a.LSE, chunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_normalize_kernel<KIND, VECTOR, EPT2>),
                     dim3(static_cast<unsigned>(a.rows * pieces)), dim3(kThreads), 0, a.stream, a.X,
                     a.Y, rowstats, a.n, pieces);
  return hipGetLastError();
}

// ---- Resident rows: one pass, slices held in registers ----
//
// A slice of SIZE consecutive elements of a row is one task; task t is part
// p = t % parts of row r = t / parts.  Workgroup b takes tasks b, b + grid,
// b + 2 grid, ... with the grid a whole number of rows, so the `parts`
// tasks of a row run in the same round.  For each task a workgroup loads the
// slice into registers as raw 16-byte words, reduces it to its (m, l),
// publishes the pair in the row's slot, waits until every slice of the row
// has published, merges the row's pairs and writes its slice of y from the
// registers: x is read from memory once.
//
// The waits complete when the whole grid is resident at once, which the
// launch arranges on an idle device (the grid is at most the kernel's
// occupancy times the CU count).  Each wait is still bounded (wait_limit
// polls): a workgroup that gives up leaves its slice unwritten, and a repair
// kernel, next on the same stream, writes every such slice from x and the
// row's pairs, which are complete by then because every task publishes
// before it waits.  So the result does not depend on residency; only the
// time does.  A slot holds its pair as one 64-bit word and l = -1 (never a
// sum of exponentials) marks it unwritten, so the pair is its own ready flag
// and no fence is needed between the publishing and the polling workgroups.
//
// Rows of more than kResidentParts slices take the two-pass form: a row's
// slowest slice holds up all of its others, and with many slices per row
// that wait costs more than the second read of x (measured on MI355X: one
// pass wins up to 32 slices a row, ties at 64 and loses beyond).
constexpr int kResidentParts = 32;

template <int KIND>
struct Slice {
  static constexpr int LOADS = 8;                       // 16-byte loads per thread
  static constexpr int EPT = LOADS * Elem<KIND>::VEC;   // 32 fp32 or 64 16-bit values
  static constexpr int SIZE = kThreads * EPT;           // elements per task
};

constexpr uint32_t kSlotPending = 0xbf800000u;   // bits of l = -1.0f

// Workspace of a resident call for T = rows * parts tasks: two counters (the
// second counts slices given up), then slots[T], then done[T] (1 once the
// slice's y is written): 16 + 12 T bytes.
struct ResidentWs {
  unsigned long long* ctr;
  unsigned long long* slots;
  unsigned* done;
};

inline ResidentWs resident_ws(void* base, int64_t tasks) {
  char* b = static_cast<char*>(base);
  ResidentWs w;
  w.ctr = reinterpret_cast<unsigned long long*>(b);
  w.slots = reinterpret_cast<unsigned long long*>(b + 16);
  w.done = reinterpret_cast<unsigned*>(b + 16 + 8 * tasks);
  return w;
}

__global__ __launch_bounds__(kThreads) void softmax_resident_clear_kernel(ResidentWs w, int64_t tasks) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < tasks; i += stride) {
    w.slots[i] = static_cast<unsigned long long>(kSlotPending) << 32;
    w.done[i] = 0u;
  }
  if (blockIdx.x == 0 && threadIdx.x < 2) w.ctr[threadIdx.x] = 0ull;
}

__device__ inline unsigned long long slot_bits(float2 ml) {
  return (static_cast<unsigned long long>(__float_as_uint(ml.y)) << 32) | __float_as_uint(ml.x);
}

__device__ inline float2 slot_pair(unsigned long long b) {
  return make_float2(__uint_as_float(static_cast<uint32_t>(b)),
                     __uint_as_float(static_cast<uint32_t>(b >> 32)));
}

__device__ inline bool slot_ready(unsigned long long b) {
  return static_cast<uint32_t>(b >> 32) != kSlotPending;
}

// One task's slice: a thread's load i covers the VEC elements from slice
// element (i * 256 + tid) * VEC on, inside the row while i * 256 + tid < kmax.
template <int KIND>
struct SliceRef {
  const u32x4* xs;
  u32x4* ys;
  int64_t r;
  int p;
  uint32_t kmax;
};

template <int KIND>
__device__ inline SliceRef<KIND> slice_of(const void* X, void* Y, int64_t n, int parts, int64_t t) {
  using E = Elem<KIND>;
  using S = Slice<KIND>;
  SliceRef<KIND> s;
  s.r = t / parts;
  s.p = static_cast<int>(t - s.r * parts);
  const int64_t start = s.r * n + static_cast<int64_t>(s.p) * S::SIZE;
  const int64_t left = n - static_cast<int64_t>(s.p) * S::SIZE;   // n is a multiple of VEC
  s.kmax = left >= S::SIZE ? S::SIZE / E::VEC : static_cast<uint32_t>(left / E::VEC);
  s.xs = reinterpret_cast<const u32x4*>(static_cast<const char*>(X) + start * E::BYTES);
  s.ys = reinterpret_cast<u32x4*>(static_cast<char*>(Y) + start * E::BYTES);
  return s;
}

template <int KIND>
__device__ inline bool in_slice(const SliceRef<KIND>& s, int i) {
  return static_cast<uint32_t>(i * kThreads) + threadIdx.x < s.kmax;
}

// Words past the row are zero; thread_pair and store_slice skip them.
template <int KIND>
__device__ inline void load_slice(const SliceRef<KIND>& s, u32x4 (&w)[Slice<KIND>::LOADS]) {
#pragma unroll
  for (int i = 0; i < Slice<KIND>::LOADS; ++i)
    w[i] = in_slice(s, i) ? Elem<KIND>::loadw(s.xs + i * kThreads + threadIdx.x, 0) : u32x4{0, 0, 0, 0};
}

// The thread's own (m, l) over its valid elements.  The empty asm statements
// keep only the packed words live between the passes over them (each pass
// unpacks again), which holds the kernel to 64 registers and so to eight
// workgroups per CU.
template <int KIND>
__device__ inline float2 thread_pair(const SliceRef<KIND>& s, u32x4 (&w)[Slice<KIND>::LOADS]) {
  constexpr int VEC = Elem<KIND>::VEC;
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < Slice<KIND>::LOADS; ++i) {
    if (in_slice(s, i)) {
      float f[VEC];
      Elem<KIND>::unpack(w[i], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) m = fmaxf(m, f[e]);
    }
  }
#pragma unroll
  for (int i = 0; i < Slice<KIND>::LOADS; ++i) asm volatile("" : "+v"(w[i]));
  float l = 0.f;
  if (m != -__builtin_inff()) {
#pragma unroll
    for (int i = 0; i < Slice<KIND>::LOADS; ++i) {
      if (in_slice(s, i)) {
        float f[VEC];
        Elem<KIND>::unpack(w[i], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) l += exp_nonpos<KIND>(f[e] - m);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < Slice<KIND>::LOADS; ++i) asm volatile("" : "+v"(w[i]));
  return make_float2(m, l);
}

template <int KIND>
__device__ inline void store_slice(const SliceRef<KIND>& s, u32x4 (&w)[Slice<KIND>::LOADS], float m,
                                   float inv) {
  using E = Elem<KIND>;
  constexpr int VEC = E::VEC;
#pragma unroll
  for (int i = 0; i < Slice<KIND>::LOADS; ++i) {
    if (in_slice(s, i)) {
      float f[VEC];
      Elem<KIND>::unpack(w[i], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = exp_nonpos<KIND>(f[e] - m) * inv;
      E::storev(s.ys + i * kThreads + threadIdx.x, 0, f);
    }
  }
}

// Polls slot *p (device-wide coherent load) until it is written or `limit`
// further polls have failed; about 0.2 us of sleep between polls.
__device__ inline bool poll_slot(const unsigned long long* p, int limit, unsigned long long& v) {
  for (int k = 0;; ++k) {
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (slot_ready(v)) return true;
    if (k >= limit) return false;
    __builtin_amdgcn_s_sleep(8);
  }
}

// X and Y may be the same buffer (in place): a slice is read in full before
// any of it is written, by the threads that write it.
template <int KIND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void
softmax_resident_kernel(const void* X, void* Y, float* __restrict__ LSE, ResidentWs ws, int64_t rows,
                        int64_t n, int parts, int wait_limit) {
  __shared__ float2 red2[4];
  const int64_t tasks = rows * parts;
  for (int64_t t = blockIdx.x; t < tasks; t += gridDim.x) {
    const SliceRef<KIND> s = slice_of<KIND>(X, Y, n, parts, t);
    u32x4 w[Slice<KIND>::LOADS];
    load_slice<KIND>(s, w);
    const float2 mine = block_merge(thread_pair<KIND>(s, w), red2);
    unsigned long long* row_slots = ws.slots + s.r * parts;
    if (threadIdx.x == 0)
      __hip_atomic_store(&row_slots[s.p], slot_bits(mine), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    float2 acc = make_float2(-__builtin_inff(), 0.f);
    for (int j = threadIdx.x; ok && j < parts; j += kThreads) {
      unsigned long long b;
      ok = poll_slot(&row_slots[j], wait_limit, b);
      if (ok) acc = merge_ml(acc, slot_pair(b));
    }
    ok = __syncthreads_and(ok);   // also ends every read of red2 above
    if (ok) {
      acc = block_merge(acc, red2);
      store_slice<KIND>(s, w, acc.x, 1.f / acc.y);
      if (threadIdx.x == 0) {
        ws.done[t] = 1u;
        if (LSE && s.p == 0) LSE[s.r] = acc.x + log_sum<KIND>(acc.y);
      }
    } else if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(&ws.ctr[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();   // red2 is written again by the next task
  }
}

// Writes the slices softmax_resident_kernel gave up on; with none (the
// usual case) every workgroup returns at once.
template <int KIND>
__global__ __launch_bounds__(kThreads) void softmax_resident_repair_kernel(
    const void* X, void* Y, float* __restrict__ LSE, ResidentWs ws, int64_t rows, int64_t n, int parts) {
  __shared__ float2 red2[4];
  if (ws.ctr[1] == 0ull) return;
  const int64_t tasks = rows * parts;
  for (int64_t t = blockIdx.x; t < tasks; t += gridDim.x) {
    if (ws.done[t]) continue;
    const SliceRef<KIND> s = slice_of<KIND>(X, Y, n, parts, t);
    u32x4 w[Slice<KIND>::LOADS];
    load_slice<KIND>(s, w);
    float2 acc = make_float2(-__builtin_inff(), 0.f);
    for (int j = threadIdx.x; j < parts; j += kThreads)
      acc = merge_ml(acc, slot_pair(ws.slots[s.r * parts + j]));
    acc = block_merge(acc, red2);
    store_slice<KIND>(s, w, acc.x, 1.f / acc.y);
    if (LSE && s.p == 0 && threadIdx.x == 0) LSE[s.r] = acc.x + log_sum<KIND>(acc.y);
    __syncthreads();
  }
}

constexpr int kWaitPollsDefault = 400;   // about 0.5 ms before a slice is given up
std::atomic<int> g_wait_polls{kWaitPollsDefault};

// Workgroups of softmax_resident_kernel<KIND> that fit on the current
// device at once (0 if that cannot be found out).
template <int KIND>
int64_t resident_capacity() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(softmax_resident_kernel<KIND>), kThreads, 0) != hipSuccess)
      per = 0;
    v = (cus > 0 && per > 0) ? cus * per : -1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

// Slices per row of the resident form, or 0 when a call takes another form.
template <int KIND>
int resident_parts(const SoftmaxArgs& a, bool vector) {
  if (!vector || a.n <= Elem<KIND>::CHUNK) return 0;
  const int64_t parts = (a.n + Slice<KIND>::SIZE - 1) / Slice<KIND>::SIZE;
  if (parts > kResidentParts || parts > resident_capacity<KIND>()) return 0;
  return static_cast<int>(parts);
}

template <int KIND>
hipError_t launch_resident(const SoftmaxArgs& a, int parts) {
  const int64_t tasks = a.rows * parts;
  const ResidentWs ws = resident_ws(a.workspace, tasks);
  const unsigned clear_grid = static_cast<unsigned>(std::min<int64_t>((tasks + kThreads - 1) / kThreads, 4096));
  hipLaunchKernelGGL(softmax_resident_clear_kernel, dim3(clear_grid), dim3(kThreads), 0, a.stream, ws, tasks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows_per_round = std::min<int64_t>(resident_capacity<KIND>() / parts, a.rows);
  hipLaunchKernelGGL((softmax_resident_kernel<KIND>), dim3(static_cast<unsigned>(rows_per_round * parts)),
                     dim3(kThreads), 0, a.stream, a.X, a.Y, a.LSE, ws, a.rows, a.n, parts,
                     g_wait_polls.load(std::memory_order_relaxed));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_resident_repair_kernel<KIND>),
                     dim3(static_cast<unsigned>(std::min<int64_t>(tasks, 256))), dim3(kThreads), 0, a.stream,
                     a.X, a.Y, a.LSE, ws, a.rows, a.n, parts);
  return hipGetLastError();
}

template <int KIND>
bool vector_rows(const SoftmaxArgs& a) {
  return (a.n % Elem<KIND>::VEC) == 0 && (reinterpret_cast<uintptr_t>(a.X) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(a.Y) % 16) == 0;
}

template <int KIND>
hipError_t launch_softmax_k(const SoftmaxArgs& a) {
  using E = Elem<KIND>;
  const bool vec = vector_rows<KIND>(a);
  if (a.n <= E::CHUNK) {
    if (vec)
      hipLaunchKernelGGL((softmax_short_kernel<KIND, true>), dim3(static_cast<unsigned>(a.rows)),
                         dim3(kThreads), 0, a.stream, a.X, a.Y, a.LSE, a.n);
    else
      hipLaunchKernelGGL((softmax_short_kernel<KIND, false>), dim3(static_cast<unsigned>(a.rows)),
                         dim3(kThreads), 0, a.stream, a.X, a.Y, a.LSE, a.n);
    return hipGetLastError();
  }
  if (const int parts = resident_parts<KIND>(a, vec)) return launch_resident<KIND>(a, parts);
  return vec ? launch_two_pass<KIND, true>(a) : launch_two_pass<KIND, false>(a);
}

template <int KIND>
int x_reads_k(const SoftmaxArgs& a) {
  if (a.n <= Elem<KIND>::CHUNK) return 1;
  return resident_parts<KIND>(a, vector_rows<KIND>(a)) ? 1 : 2;
}

}  // namespace

int64_t softmax_chunk(int dtype) { return dtype == kDtypeF32 ? Elem<0>::CHUNK : Elem<2>::CHUNK; }
int64_t softmax_slice(int dtype) { return dtype == kDtypeF32 ? Slice<0>::SIZE : Slice<2>::SIZE; }
int64_t softmax_piece(int dtype) {
  return dtype == kDtypeF32 ? int64_t{kThreads} * Elem<0>::VEC : int64_t{kThreads} * Elem<2>::VEC;
}

hipError_t launch_softmax(const SoftmaxArgs& a) {
  if (a.dtype == kDtypeBF16) return launch_softmax_k<2>(a);
  if (a.dtype == kDtypeF16) return launch_softmax_k<1>(a);
  return launch_softmax_k<0>(a);
}

int softmax_x_reads(const SoftmaxArgs& a) {
  if (a.dtype == kDtypeBF16) return x_reads_k<2>(a);
  if (a.dtype == kDtypeF16) return x_reads_k<1>(a);
  return x_reads_k<0>(a);
}

int softmax_wait_limit(int polls) {
  return g_wait_polls.exchange(polls < 0 ? kWaitPollsDefault : polls, std::memory_order_relaxed);
}

}  // namespace iofa
