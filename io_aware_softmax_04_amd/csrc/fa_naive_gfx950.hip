// Naive three-kernel attention for gfx950: the standard-attention contrast
// whose device-memory traffic section "MAC分析 / 标准Transformer MAC分析" of
// the ctyun.cn FlashAttention article counts step by step:
//   kernel 1: read Q, K; write S = scale * Q K^T        (2Nd + N^2 elements)
//   kernel 2: read S; write P = softmax(S) row by row  (2N^2)
//   kernel 3: read P, V; write O = P V                  (N^2 + 2Nd)
// S and P are stored in the input element type with row stride ldS (N
// rounded up to 8, so each row starts 16-byte aligned); kernel 2 writes
// zeros into P's padding columns, so kernel 3 can read whole 8-key chunks.
// The matrix products of 16-bit inputs use v_mfma_f32_32x32x16 with fp32
// accumulation; fp32 inputs use plain fp32 FMAs.
#include "fa_device.h"
#include "fa_launch.h"

namespace iofa {

namespace {

constexpr int kQRows = 128;        // query rows per workgroup (4 waves x 32)
constexpr int kKeysPerWg = 256;    // keys per workgroup in kernel 1
constexpr int kMaxChunks = 16;     // 8-element chunks per thread in kernel 2 (N <= 32768)
// S and P are written with streaming (non-temporal) stores when one of them is
// larger than the 256 MB last-level cache (MALL): there the next kernel's
// reads miss it anyway, and streaming stores took the path at B2 H16 N4096
// d128 (1 GiB each) from 952 to 882 us, 6% at N = 8191.  Smaller ones keep
// normal stores, which leave them in the MALL for the next kernel (streaming
// stores made B4 H16 N1024 d64, 128 MiB each, 5% slower).
constexpr uint64_t kStreamBytes = uint64_t(256) << 20;
// cache-policy operand of a buffer store: non-temporal
constexpr int kCpolNT = 2;

// K tile of BC rows x D 16-bit elements into LDS rows of stride KS elements
// (kernel 1).  256 threads; each owns KCH 16-byte chunks; consecutive threads
// read consecutive chunks of one row (coalesced).  The loads are range-checked
// buffer loads over the tile's valid rows, so rows at or beyond `rows_valid`
// arrive as zeros without a branch, and the compiler can count them exactly
// in its waits.
template <int D, int BC, int KS>
struct RowTile {
  static constexpr int CH = D / 8;
  static constexpr int KCH = BC * CH / 256;
  static_assert(KCH * 256 == BC * CH, "tile must split into 256 threads");
  u32x4 r[KCH];

  __device__ inline void load(const uint16_t* __restrict__ base, int rows_valid, int tid) {
    // workgroup-uniform: keeps the buffer descriptor in scalar registers
    const int rows = __builtin_amdgcn_readfirstlane(rows_valid > 0 ? (rows_valid < BC ? rows_valid : BC) : 0);
    const auto rsrc = buffer_rsrc(base, static_cast<uint32_t>(rows) * (D * 2u));
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, cc = c % CH;
      r[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (row * D + cc * 8) * 2, 0, 0));
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, cc = c % CH;
      *reinterpret_cast<u32x4*>(lds + row * KS + cc * 8) = r[i];
    }
  }
};

// ------------------------------------------------ element access (kernel 2)

struct Ld16Bf16 {
  __device__ static inline float to_f32(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static inline uint16_t from_f32(float x) { return Bf16::bits(x); }
  __device__ static inline float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
};
struct Ld16F16 {
  __device__ static inline float to_f32(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  __device__ static inline uint16_t from_f32(float x) { return F16::bits(x); }
  __device__ static inline float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
};

template <class E>
__device__ inline void load8_16(const uint16_t* p, float* v) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = E::to_f32(half_of(w, e));
}
template <class E, bool STREAM>
__device__ inline void store8_16(uint16_t* p, const float* v) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack2(E::from_f32(v[2 * e]), E::from_f32(v[2 * e + 1]));
  if constexpr (STREAM) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = w;
}

__device__ inline float block_reduce(float x, bool is_max, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float y = __shfl_xor(x, off, 64);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// ------------------------------------------------------- kernel 1 (16-bit)

template <class T, int D, bool STREAM>
__global__ __launch_bounds__(256, 4) void naive_scores_16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    uint16_t* __restrict__ S, int N, int ldS, int qtiles, int ktiles, int num_wg,
    float scale) {
  constexpr int BC = 64, KS = D + 8, SS = BC + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Ss[kQRows * SS];   // one S block
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int bh = L / (qtiles * ktiles);
  const int rem = L % (qtiles * ktiles);
  const int qt = rem / ktiles, kt = rem % ktiles;
  const size_t head = static_cast<size_t>(bh) * N * D;

  const int q = qt * kQRows + wave * 32 + l32;
  typename T::vec8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = (q < N) ? gmem_vec8<T>(Q + head + static_cast<size_t>(q) * D + 16 * kk + 8 * hi)
                     : __builtin_bit_cast(typename T::vec8, u32x4{0u, 0u, 0u, 0u});
  // The K rows of the next 64-key block are loaded while this block is
  // multiplied and its scores are stored, so the wait for them (which on
  // this GPU also waits for every store issued before them) never waits for
  // the current block's stores.
  RowTile<D, BC, KS> t;
  {
    const int k0 = kt * kKeysPerWg;
    t.load(K + head + static_cast<size_t>(k0) * D, N - k0, tid);
  }
#pragma unroll
  for (int sub = 0; sub < kKeysPerWg / BC; ++sub) {
    const int k0 = kt * kKeysPerWg + sub * BC;
    if (k0 >= N) break;
    t.store(Ks, tid);
    __syncthreads();
    const int k1 = k0 + BC;
    if (sub + 1 < kKeysPerWg / BC) t.load(K + head + static_cast<size_t>(k1) * D, N - k1, tid);
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
        s[sb] = T::mfma(lds_vec8<T>(Ks + (32 * sb + l32) * KS + 16 * kk + 8 * hi), qf[kk], s[sb]);
    // the block's scores (query rows x 64 keys) go through LDS so that each
    // row is written as contiguous 16-byte pieces
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack2(T::bits(s[sb][4 * g + 0] * scale), T::bits(s[sb][4 * g + 1] * scale));
        w[1] = pack2(T::bits(s[sb][4 * g + 2] * scale), T::bits(s[sb][4 * g + 3] * scale));
        *reinterpret_cast<u32x2*>(Ss + (wave * 32 + l32) * SS + 32 * sb + 8 * g + 4 * hi) = w;
      }
    __syncthreads();
    constexpr int CPR = BC / 8;                         // 16-byte pieces per row
    // Range-checked buffer stores over the workgroup's valid rows of S: a
    // piece outside them (a row at or beyond N, or a key at or beyond ldS)
    // gets an offset past the range and is dropped.  Being branch-free, the
    // stores are counted exactly by the compiler's waits, so the next
    // block's K loads (issued before them) are waited for without them.
    // ldS is a multiple of 8, so a piece that starts before ldS ends there at
    // the latest; columns in [N, ldS) are never read as scores.
    const int qrows = N - qt * kQRows < kQRows ? N - qt * kQRows : kQRows;
    const uint32_t sbytes = static_cast<uint32_t>(qrows) * static_cast<uint32_t>(ldS) * 2u;
    const auto srsrc = buffer_rsrc(S + (static_cast<size_t>(bh) * N + qt * kQRows) * ldS, sbytes);
#pragma unroll
    for (int i = 0; i < kQRows * CPR / 256; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CPR, key = k0 + 8 * (c % CPR);
      const uint32_t off = (r < qrows && key < ldS)
                               ? (static_cast<uint32_t>(r) * ldS + key) * 2u : sbytes;
      __builtin_amdgcn_raw_buffer_store_b128(
          *reinterpret_cast<const u32x4*>(Ss + r * SS + 8 * (c % CPR)),
          srsrc, static_cast<int>(off), 0, STREAM ? kCpolNT : 0);
    }
    __syncthreads();
  }
}

// --------------------------------------------------------- kernel 2 (all)

// MAXC: 8-element chunks per thread the row needs (a power of two, at most
// kMaxChunks); instances for short rows hold fewer registers, so more rows
// are in flight per CU.
template <class E, int MAXC, bool STREAM>
__global__ __launch_bounds__(256) void naive_softmax_16(
    const uint16_t* __restrict__ S, uint16_t* __restrict__ P, float* __restrict__ LSE,
    int N, int ldS) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const uint16_t* s = S + row * ldS;
  uint16_t* p = P + row * ldS;
  const int nch = ldS / 8;
  float v[MAXC][8];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      load8_16<E>(s + c * 8, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (c * 8 + e >= N) v[i][e] = -__builtin_inff();
        mx = fmaxf(mx, v[i][e]);
      }
    }
  }
  mx = block_reduce(mx, true, red);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = E::ex(v[i][e] - mx);
        sum += v[i][e];
      }
    }
  }
  sum = block_reduce(sum, false, red);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = v[i][e] * inv;
      store8_16<E, STREAM>(p + c * 8, w);
    }
  }
  if (LSE != nullptr && threadIdx.x == 0) LSE[row] = mx + logf(sum);
}

__global__ __launch_bounds__(256) void naive_softmax_f32(
    const float* __restrict__ S, float* __restrict__ P, float* __restrict__ LSE, int N,
    int ldS) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const float* s = S + row * ldS;
  float* p = P + row * ldS;
  const int nch = ldS / 8;
  float v[kMaxChunks][8];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      const float4 a = *reinterpret_cast<const float4*>(s + c * 8);
      const float4 b = *reinterpret_cast<const float4*>(s + c * 8 + 4);
      v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
      v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (c * 8 + e >= N) v[i][e] = -__builtin_inff();
        mx = fmaxf(mx, v[i][e]);
      }
    }
  }
  mx = block_reduce(mx, true, red);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = expf(v[i][e] - mx);
        sum += v[i][e];
      }
    }
  }
  sum = block_reduce(sum, false, red);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      *reinterpret_cast<float4*>(p + c * 8) =
          make_float4(v[i][0] / sum, v[i][1] / sum, v[i][2] / sum, v[i][3] / sum);
      *reinterpret_cast<float4*>(p + c * 8 + 4) =
          make_float4(v[i][4] / sum, v[i][5] / sum, v[i][6] / sum, v[i][7] / sum);
    }
  }
  if (LSE != nullptr && threadIdx.x == 0) LSE[row] = mx + logf(sum);
}

// ------------------------------------------------------- kernel 3 (16-bit)

// O = P V for 128 query rows per workgroup (32 per wave), 64-key tiles.
// Each lane holds one query row's P fragments (8 consecutive keys, straight
// from global memory, the MFMA's B operand); V tiles are copied into LDS
// with direct buffer loads (row-major, chunks swizzled as for the fused
// kernel's V) and read back transposed with ds_read_b64_tr_b16 as the A
// operand, so V needs neither staging registers nor transposing stores.
// Iteration j issues the loads of tile j+1 (P into registers, V into the
// other LDS stage) before multiplying tile j, and ends with a wait for them
// and a barrier.
template <class T, int D>
__global__ __launch_bounds__(256, 4) void naive_pv_16(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, int N, int ldS, int qtiles, int num_wg) {
  constexpr int BC = 64;
  constexpr uint32_t TB = BC * D * 2u;                 // bytes of one V stage
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * BC * D];
  const uint32_t sm = lds_address(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int bh = L / qtiles, qt = L % qtiles;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int q = qt * kQRows + wave * 32 + l32;
  const uint16_t* Prow = P + (static_cast<size_t>(bh) * N + q) * ldS;

  // V^T fragments: in each 16-lane group (g = lane / 16, t = lane % 16) lane
  // t supplies row 8*(g/2) + t/4 and columns c0 + 4*(t%4) .. +3 and receives
  // column c0 + t of 4 consecutive rows; the second read is 4 rows further.
  // Lane half hi thus gets keys 16*ks + 8*hi + 0..7, the keys its P
  // fragment holds.  The swizzle depends on row % 4 only.
  uint32_t v_addr[D / 32];
  {
    const int g = lane >> 4, t = lane & 15;
    const int row = 8 * (g >> 1) + (t >> 2);
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int col = 32 * cb + 16 * (g & 1) + 4 * (t & 3);
      const int chunk = (col >> 3) ^ v_swz<D>(row);
      v_addr[cb] = sm + static_cast<uint32_t>(row * D + chunk * 8 + (col & 7)) * 2u;
    }
  }
  TileCopy<D, BC, kSwzV> vcp;
  vcp.init(wave, lane);

  using vec8 = typename T::vec8;
  auto load_p = [&](int k0, vec8 (&pf)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kidx = k0 + 16 * ks + 8 * hi;
      pf[ks] = (q < N && kidx < ldS) ? gmem_vec8<T>(Prow + kidx)
                                     : __builtin_bit_cast(vec8, u32x4{0u, 0u, 0u, 0u});
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) o[cb] = f32x16{};
  const int NT = (N + BC - 1) / BC;
  vec8 pcur[4], pnext[4];
  load_p(0, pcur);
  vcp.copy(V + head, 0, N, sm);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j < NT; ++j) {
    const uint32_t cur = (j & 1) ? TB : 0u;
    if (j + 1 < NT) {
      load_p((j + 1) * BC, pnext);
      vcp.copy(V + head, (j + 1) * BC, N, sm + (TB - cur));
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const uint32_t a0 = v_addr[cb] + cur + 16u * ks * D * 2u;
        const s16x4 lo = lds_read_tr8(a0);
        const s16x4 up = lds_read_tr8(a0 + 4u * D * 2u);
        const auto a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        o[cb] = T::mfma(a, pcur[ks], o[cb]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pcur[ks] = pnext[ks];
  }
  if (q < N) {
    uint16_t* Oq = O + head + static_cast<size_t>(q) * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack2(T::bits(o[cb][4 * g + 0]), T::bits(o[cb][4 * g + 1]));
        w[1] = pack2(T::bits(o[cb][4 * g + 2]), T::bits(o[cb][4 * g + 3]));
        *reinterpret_cast<u32x2*>(Oq + 32 * cb + 8 * g + 4 * hi) = w;
      }
  }
}

// --------------------------------------------------- kernels 1, 3 (fp32)

// One thread per score; 16 x 16 score tile per workgroup.
__global__ __launch_bounds__(256) void naive_scores_f32(
    const float* __restrict__ Q, const float* __restrict__ K, float* __restrict__ S,
    int N, int D, int ldS, int tiles, float scale) {
  const int per_head = tiles * tiles;
  const int bh = blockIdx.x / per_head, t = blockIdx.x % per_head;
  const int i = (t / tiles) * 16 + threadIdx.x / 16;
  const int j = (t % tiles) * 16 + threadIdx.x % 16;
  if (i >= N || j >= N) return;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const float* qi = Q + head + static_cast<size_t>(i) * D;
  const float* kj = K + head + static_cast<size_t>(j) * D;
  float acc = 0.f;
  for (int c = 0; c < D; ++c) acc = fmaf(qi[c], kj[c], acc);
  S[(static_cast<size_t>(bh) * N + i) * ldS + j] = acc * scale;
}

// One thread per output element.
__global__ __launch_bounds__(256) void naive_pv_f32(
    const float* __restrict__ P, const float* __restrict__ V, float* __restrict__ O,
    int N, int D, int ldS, int64_t total) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % D);
  const int64_t rowg = idx / D;  // bh * N + i
  const int64_t bh = rowg / N;
  const float* prow = P + rowg * ldS;
  const float* vh = V + bh * N * D;
  float acc = 0.f;
  for (int j = 0; j < N; ++j) acc = fmaf(prow[j], vh[static_cast<size_t>(j) * D + c], acc);
  O[idx] = acc;
}

// ---------------------------------------------------------------- launch

template <class E, int MAXC, bool STREAM>
hipError_t launch_naive_softmax16_c(const NaiveArgs& a, int N, int ldS) {
  hipLaunchKernelGGL((naive_softmax_16<E, MAXC, STREAM>), dim3(static_cast<unsigned>(a.f.BH * N)),
                     dim3(256), 0, a.f.stream, static_cast<const uint16_t*>(a.S),
                     static_cast<uint16_t*>(a.P), a.f.LSE, N, ldS);
  return hipGetLastError();
}

template <class E, bool STREAM>
hipError_t launch_naive_softmax16(const NaiveArgs& a, int N, int ldS) {
  const int per_thread = (ldS / 8 + 255) / 256;   // chunks per thread the row needs
  if (per_thread <= 1) return launch_naive_softmax16_c<E, 1, STREAM>(a, N, ldS);
  if (per_thread <= 2) return launch_naive_softmax16_c<E, 2, STREAM>(a, N, ldS);
  if (per_thread <= 4) return launch_naive_softmax16_c<E, 4, STREAM>(a, N, ldS);
  if (per_thread <= 8) return launch_naive_softmax16_c<E, 8, STREAM>(a, N, ldS);
  return launch_naive_softmax16_c<E, kMaxChunks, STREAM>(a, N, ldS);
}

template <class T, class E, int D, bool STREAM>
hipError_t launch_naive16_s(const NaiveArgs& a) {
  const FwdArgs& f = a.f;
  const int N = static_cast<int>(f.N), ldS = static_cast<int>(a.ldS);
  const int qtiles = (N + kQRows - 1) / kQRows;
  const int ktiles = (N + kKeysPerWg - 1) / kKeysPerWg;
  const int wg1 = static_cast<int>(f.BH * qtiles * ktiles);
  hipLaunchKernelGGL((naive_scores_16<T, D, STREAM>), dim3(wg1), dim3(256), 0, f.stream,
                     static_cast<const uint16_t*>(f.Q), static_cast<const uint16_t*>(f.K),
                     static_cast<uint16_t*>(a.S), N, ldS, qtiles, ktiles, wg1, f.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_naive_softmax16<E, STREAM>(a, N, ldS);
  if (e != hipSuccess) return e;
  const int wg3 = static_cast<int>(f.BH * qtiles);
  hipLaunchKernelGGL((naive_pv_16<T, D>), dim3(wg3), dim3(256), 0, f.stream,
                     static_cast<const uint16_t*>(a.P), static_cast<const uint16_t*>(f.V),
                     static_cast<uint16_t*>(f.O), N, ldS, qtiles, wg3);
  return hipGetLastError();
}

template <class T, class E, int D>
hipError_t launch_naive16(const NaiveArgs& a) {
  const uint64_t s_bytes = static_cast<uint64_t>(a.f.BH) * static_cast<uint64_t>(a.f.N) *
                           static_cast<uint64_t>(a.ldS) * 2u;
  return s_bytes > kStreamBytes ? launch_naive16_s<T, E, D, true>(a)
                                : launch_naive16_s<T, E, D, false>(a);
}

hipError_t launch_naive32(const NaiveArgs& a) {
  const FwdArgs& f = a.f;
  const int N = static_cast<int>(f.N), D = static_cast<int>(f.d), ldS = static_cast<int>(a.ldS);
  const int tiles = (N + 15) / 16;
  hipLaunchKernelGGL(naive_scores_f32, dim3(static_cast<unsigned>(f.BH * tiles * tiles)), dim3(256),
                     0, f.stream, static_cast<const float*>(f.Q), static_cast<const float*>(f.K),
                     static_cast<float*>(a.S), N, D, ldS, tiles, f.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(naive_softmax_f32, dim3(static_cast<unsigned>(f.BH * N)), dim3(256), 0,
                     f.stream, static_cast<const float*>(a.S), static_cast<float*>(a.P), f.LSE, N,
                     ldS);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = f.BH * N * D;
  hipLaunchKernelGGL(naive_pv_f32, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                     f.stream, static_cast<const float*>(a.P), static_cast<const float*>(f.V),
                     static_cast<float*>(f.O), N, D, ldS, total);
  return hipGetLastError();
}

}  // namespace

int64_t naive_max_workgroups(int dtype, int64_t BH, int64_t N) {
  if (dtype == kDtypeF32) {
    const int64_t tiles = (N + 15) / 16;
    const int64_t a = BH * tiles * tiles, b = BH * N, c = (BH * N * 128 + 255) / 256;
    return a > b ? (a > c ? a : c) : (b > c ? b : c);
  }
  const int64_t qt = (N + kQRows - 1) / kQRows, kt = (N + kKeysPerWg - 1) / kKeysPerWg;
  const int64_t a = BH * qt * kt, b = BH * N;
  return a > b ? a : b;
}

hipError_t launch_naive(const NaiveArgs& a) {
  const int dt = a.f.dtype;
  const bool d128 = a.f.d == 128;
  if (dt == kDtypeBF16)
    return d128 ? launch_naive16<Bf16, Ld16Bf16, 128>(a) : launch_naive16<Bf16, Ld16Bf16, 64>(a);
  if (dt == kDtypeF16)
    return d128 ? launch_naive16<F16, Ld16F16, 128>(a) : launch_naive16<F16, Ld16F16, 64>(a);
  return launch_naive32(a);
}

}  // namespace iofa
