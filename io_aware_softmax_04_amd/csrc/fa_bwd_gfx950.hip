// Backward pass of exact attention for gfx950 (16-bit inputs).
//
// xinc.fun archive 235, section "7. Online Softmax", closes with the point
// that the backward pass recomputes local scores from the saved inputs and a
// few statistics instead of reading a stored attention matrix.  With the
// forward's log-sum-exp L (natural log, scaled scores) every tile of
// P = exp(scale * Q K^T - L) is rebuilt on chip, and for an upstream dO:
//     D_i = sum_c dO_ic O_ic,   dS = P * (dO V^T - D),
//     dV = P^T dO,   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Three kernels:
//   bwd_stats    per row: (L * log2 e, -D) into an fp32 pair workspace;
//   bwd_dq       one workgroup per 128 query rows (4 waves x 32), K and V
//                tiles of 32 keys streamed through LDS; per tile
//                S^T = K Q^T, dP^T = V dO^T (both v_mfma_f32_32x32x16 with
//                the lane owning a query column), P^T and dS^T in-lane,
//                dQ^T += K^T dS^T with dS^T straight from registers and K^T
//                read through ds_read_b64_tr_b16 -- the shape of the fused
//                forward's P V; software-pipelined across tiles like the
//                forward (see the kernel);
//   bwd_dkdv     one workgroup per 128 keys (4 waves x 32), Q and dO tiles
//                of 32 queries (with their (L log2 e, D) pairs) streamed;
//                per tile S = Q K^T and dP = dO V^T with the lane owning a
//                key column (K fragments in registers, the workgroup's V
//                rows resident in LDS), then dV^T += dO^T P and
//                dK^T += Q^T dS with P, dS from registers and dO^T, Q^T
//                through transposed reads.
// dQ and dK recompute S and dP separately (7 products of N^2 d per head
// against the 5 a single pass with atomic dQ updates would need) so that no
// output is shared between workgroups and the result is deterministic.
// Tiles that are read both as row fragments and transposed use the kv_swz
// swizzle; copies are buffer_load ... lds into LDS stages with later tiles'
// copies in flight while the current one is computed; the tile loops are
// unrolled (by four in bwd_dq, by two in bwd_dkdv) so stage offsets are
// immediates.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace iofa {

namespace {

constexpr int kBwdTile = 32;                 // keys (dq) / queries (dkdv) per tile
constexpr int kBwdRows = 128;                // rows a workgroup owns (4 waves x 32)

// ------------------------------------------------------------- stats pass

// (L[r] * log2 e, -D[r]) for every row r of B*H*N.  D/8 threads per row, each
// 8 columns (16-byte loads).  D enters dS = P (dP - D) negated, so the dK/dV
// kernel can start its dP accumulator from it.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const uint16_t* __restrict__ O,
                                                        const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        float2* __restrict__ stats, int64_t rows) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int c8 = threadIdx.x % TPR;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(O + r * D + 8 * c8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + r * D + 8 * c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(T::to_f32(half_of(o, e)), T::to_f32(half_of(g, e)), acc);
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (r < rows && c8 == 0) stats[r] = make_float2(LSE[r] * kLog2e, -acc);
}

// ------------------------------------------------------------ shared steps

// Per-lane LDS byte offsets (relative to a stage) of the two read patterns of
// a kv_swz-swizzled tile of 32 rows, computed once so that every read in the
// loop is a register plus an immediate (the stage offset).
template <int D>
struct LaneOffsets {
  uint32_t row[D / 16];     // row fragment: row l32, chunk 2*kk + hi
  uint32_t col[D / 32][2];  // transposed read: rows row0 (+8), columns 32*cb + ...

  __device__ inline void init(int lane, int row_base) {
    const int l32 = lane & 31, hi = lane >> 5;
    const int r = row_base + l32;
    const int swz = kv_swz<D>(r);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      row[kk] = static_cast<uint32_t>(r * D + (((2 * kk + hi) ^ swz) * 8)) * 2u;
    const int g = lane >> 4, t = lane & 15;
    const int row0 = 4 * (g >> 1) + (t >> 2);
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int rr = row0 + 8 * h8;
        const int c = 32 * cb + 16 * (g & 1) + 4 * (t & 3);
        const int chunk = (c >> 3) ^ kv_swz<D>(rr);
        col[cb][h8] = static_cast<uint32_t>(rr * D + chunk * 8 + (c & 7)) * 2u;
      }
  }
};

// Row-fragment product: acc (32 x 32) += A (32 rows of an LDS tile, all D
// columns; lane (l32, hi) reads row l32, chunk 2*kk + hi) times B (D x 32,
// per-lane fragments bf[kk]).
template <class T, int D>
__device__ inline void rows_times(f32x16& acc, uint32_t base, const LaneOffsets<D>& lo,
                                  const typename T::vec8 (&bf)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    acc = T::mfma(__builtin_bit_cast(typename T::vec8, lds_read16(base + lo.row[kk])), bf[kk], acc);
}

// The same product with B's fragments read from another LDS tile of the same
// layout (lane (l32, hi) holds row l32, columns 16*kk + 8*hi .. +7), one
// k-step at a time so that no whole operand is held in registers.
template <class T, int D>
__device__ inline void rows_times_lds(f32x16& acc, uint32_t abase, uint32_t bbase,
                                      const LaneOffsets<D>& lo) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    acc = T::mfma(__builtin_bit_cast(typename T::vec8, lds_read16(abase + lo.row[kk])),
                  __builtin_bit_cast(typename T::vec8, lds_read16(bbase + lo.row[kk])), acc);
}

// Transposed-fragment product: out[cb] (32 columns c x 32) += A^T (columns
// 32*cb.. of a 32-row LDS tile, rows = the product's k index) times the
// packed B fragments pk[ks] (k-slot 8*hi + u of step ks holds tile row
// 16*ks + 8*(u/4) + 4*hi + u%4, the order of an MFMA accumulator's rows).
template <class T, int D>
__device__ inline void cols_times(f32x16 (&out)[D / 32], uint32_t base, const LaneOffsets<D>& lo,
                                  const typename T::vec8 (&pk)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const s16x4 lo4 = lds_read_tr8(base + lo.col[cb][0] + 16 * ks * D * 2);
      const s16x4 up4 = lds_read_tr8(base + lo.col[cb][1] + 16 * ks * D * 2);
      const auto a = __builtin_bit_cast(typename T::vec8,
                                        __builtin_shufflevector(lo4, up4, 0, 1, 2, 3, 4, 5, 6, 7));
      out[cb] = T::mfma(a, pk[ks], out[cb]);
    }
  }
}

// Pack 32 fp32 accumulator values (two 16-register halves) into the two
// k-step B fragments of a product over the accumulator's rows.
template <class T>
__device__ inline void pack_b(const f32x16& v, typename T::vec8 (&pk)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = T::pack(v[8 * ks + 2 * e], v[8 * ks + 2 * e + 1]);
    pk[ks] = __builtin_bit_cast(typename T::vec8, w);
  }
}

// Stores a transposed accumulator out[cb] (lane = row of the output, its
// registers = columns 32*cb + 8*g + 4*hi + 0..3) times `mul`, rounded.
template <class T, int D>
__device__ inline void store_rowmajor(uint16_t* dst, const f32x16 (&out)[D / 32], int hi, float mul) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = T::pack(out[cb][4 * g + 0] * mul, out[cb][4 * g + 1] * mul);
      w[1] = T::pack(out[cb][4 * g + 2] * mul, out[cb][4 * g + 3] * mul);
      *reinterpret_cast<u32x2*>(dst + 32 * cb + 8 * g + 4 * hi) = w;
    }
  }
}

template <class T, int D>
__device__ inline void load_row_frags(typename T::vec8 (&f)[D / 16], const uint16_t* row, bool valid,
                                      int hi) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (valid) w = *reinterpret_cast<const u32x4*>(row + 16 * kk + 8 * hi);
    f[kk] = __builtin_bit_cast(typename T::vec8, w);
  }
}

using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

// --------------------------------------------------------------- dQ kernel
//
// Per wave (32 query rows) and 32-key tile t: S^T_t and dP^T_t (MFMA), then
// P_t and dS_t (vector unit), then dQ^T += K_t^T dS^T_t (MFMA).  The loop is
// software-pipelined like the fused forward: iteration j computes P_j, dS_j
// while the matrix cores run dQ for tile j-1 and S^T, dP^T for tile j+1.  K
// tile t is read in iterations t-1 (scores) and t+1 (transposed, for dQ) and
// copied in iteration t-2, so K has four LDS stages; V tile t is read in
// iteration t-1 only (two stages).  Score and dP registers alternate between
// two sets by tile parity; the loop is unrolled by four so every stage offset
// is an immediate.

template <class T, int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float2* __restrict__ stats, uint16_t* __restrict__ dQ, int N, int num_qtiles,
    int num_wg, float scale) {
  using vec8 = typename T::vec8;
  constexpr int BC = kBwdTile;
  constexpr uint32_t TB = BC * D * 2u;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[6 * BC * D];   // K0..K3 V0 V1
  const uint32_t sm = lds_address(smem);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;

  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int bh = L / num_qtiles, qt = L % num_qtiles;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int q = qt * kBwdRows + wave * 32 + l32;
  const bool qv = q < N;
  TileCopy<D, BC, kSwzKV> kcp;
  TileCopy<D, BC, kSwzKV> vcp;
  kcp.init(wave, lane);
  vcp.init(wave, lane);
  LaneOffsets<D> lo;
  lo.init(lane, 0);
  const int NT = (N + BC - 1) / BC;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  auto copy_tile = [&](int t) {   // K_t -> K stage t % 4, V_t -> V stage t % 2
    kcp.copy(Kh, t * BC, N, sm + (t & 3) * TB);
    vcp.copy(Vh, t * BC, N, sm + (4 + (t & 1)) * TB);
  };
  copy_tile(0);
  if (NT > 1) copy_tile(1);

  vec8 qf[D / 16], df[D / 16];
  load_row_frags<T, D>(qf, Q + head + static_cast<size_t>(q) * D, qv, hi);
  load_row_frags<T, D>(df, dO + head + static_cast<size_t>(q) * D, qv, hi);
  const float2 st = qv ? stats[static_cast<size_t>(bh) * N + q] : make_float2(0.f, 0.f);
  const float lse2 = st.x, negD = st.y;
  // dP^T starts from -D (the lane's query), so it ends as dP - D and dS is one
  // multiply per element; the first dP product reads this block as its
  // accumulator input, so the start costs no vector instruction per tile
  f32x16 nd16;
#pragma unroll
  for (int r = 0; r < 16; ++r) nd16[r] = negD;
  const float c2 = scale * kLog2e;
  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};

  // score / dP register sets by tile parity, packed dS by tile parity
  f32x16 s_[2], dp_[2];
  vec8 pk_[2][2];

  // S^T_t, dP^T_t into set t % 2 (K stage KS, V stage VS)
  auto scores = [&](auto set, auto ks, auto vs) {
    constexpr int SET = decltype(set)::value, KS = decltype(ks)::value, VS = decltype(vs)::value;
    s_[SET] = f32x16{};
    dp_[SET] = nd16;
    rows_times<T, D>(s_[SET], sm + KS * TB, lo, qf);          // S^T  (keys x queries)
    rows_times<T, D>(dp_[SET], sm + (4 + VS) * TB, lo, df);   // dP^T
  };
  // P_t, dS_t of set SET, packed; TAIL masks keys at or beyond kvalid
  auto softmax_ds = [&](auto set, auto tail, int kvalid) {
    constexpr int SET = decltype(set)::value;
    constexpr bool TAIL = decltype(tail)::value;
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(fmaf(s_[SET][r], c2, -lse2));
      if (TAIL) {
        const int key = 8 * (r >> 2) + 4 * hi + (r & 3);
        p = key < kvalid ? p : 0.f;
      }
      ds[r] = p * dp_[SET][r];
    }
    pack_b<T>(ds, pk_[SET]);
  };
  // dQ^T += K_t^T dS^T_t, K_t in stage KS, dS_t in set SET
  auto dq_update = [&](auto set, auto ks) {
    constexpr int SET = decltype(set)::value, KS = decltype(ks)::value;
    cols_times<T, D>(acc, sm + KS * TB, lo, pk_[SET]);
  };
  auto bottom = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using NoTail = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  constexpr int NM = 3 * (D / 16);                 // products per middle iteration
  constexpr int NRD = 2 * (D / 16) + 2 * (D / 16); // 2 b128 per score step, 2 transposed per dQ step

  // middle iteration j (0 < j < NT-1), J = j % 4
  auto middle = [&](auto jm, int j) {
    constexpr int J = decltype(jm)::value;
    using Cur = std::integral_constant<int, J % 2>;
    using Nxt = std::integral_constant<int, (J + 1) % 2>;
    // raised issue priority through the products, dropped before the
    // barrier, as in the forward kernels
    __builtin_amdgcn_s_setprio(1);
    if (j + 2 < NT) copy_tile(j + 2);
    softmax_ds(Cur{}, NoTail{}, BC);
    dq_update(Nxt{}, std::integral_constant<int, (J + 3) % 4>{});    // tile j-1
    scores(Nxt{}, std::integral_constant<int, (J + 1) % 4>{},
           std::integral_constant<int, (J + 1) % 2>{});             // tile j+1
    interleave_mfma_valu<NM, NRD, 8, 3>();
    __builtin_amdgcn_s_setprio(0);
    bottom();
  };
  // last iteration j = NT-1 (> 0), J = j % 4: no copies, no scores
  auto last = [&](auto jm, int j) {
    constexpr int J = decltype(jm)::value;
    using Cur = std::integral_constant<int, J % 2>;
    using Prv = std::integral_constant<int, (J + 1) % 2>;
    softmax_ds(Cur{}, Tail{}, N - j * BC);
    dq_update(Prv{}, std::integral_constant<int, (J + 3) % 4>{});    // tile j-1
    dq_update(Cur{}, std::integral_constant<int, J>{});              // tile j
  };

  bottom();                                        // tiles 0 and 1 are in LDS
  scores(I0{}, I0{}, I0{});                        // tile 0
  if (NT == 1) {
    softmax_ds(I0{}, Tail{}, N);
    dq_update(I0{}, I0{});
  } else {
    // iteration 0: P_0, dS_0 with the scores of tile 1
    if (NT > 2) copy_tile(2);
    softmax_ds(I0{}, NoTail{}, BC);
    scores(I1{}, I1{}, I1{});
    interleave_mfma_valu<2 * (D / 16), 2 * (D / 16), 4, 3>();
    bottom();
    int j = 1;
    for (; j + 4 <= NT - 1; j += 4) {
      middle(I1{}, j);
      middle(I2{}, j + 1);
      middle(I3{}, j + 2);
      middle(I0{}, j + 3);
    }
    // j % 4 == 1 here; at most three middle iterations remain
    if (j < NT - 1) { middle(I1{}, j); ++j; }
    if (j < NT - 1) { middle(I2{}, j); ++j; }
    if (j < NT - 1) { middle(I3{}, j); ++j; }
    switch (j & 3) {
      case 0: last(I0{}, j); break;
      case 1: last(I1{}, j); break;
      case 2: last(I2{}, j); break;
      default: last(I3{}, j); break;
    }
  }
  if (qv) store_rowmajor<T, D>(dQ + head + static_cast<size_t>(q) * D, acc, hi, scale);
  __builtin_amdgcn_s_waitcnt(0);
}

// ------------------------------------------------------------ dK/dV kernel

template <class T, int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float2* __restrict__ stats, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N,
    int num_ktiles, int num_wg, float scale) {
  using vec8 = typename T::vec8;
  constexpr int BQ = kBwdTile;
  constexpr uint32_t TB = BQ * D * 2u;
  constexpr uint32_t SB = BQ * 8u;                       // (lse2, D) pairs of a tile
  constexpr uint32_t VB = kBwdRows * D * 2u;             // the workgroup's V rows
  // Q0 Q1 dO0 dO1 (TB each), stats 0, 1 (SB each), then V (VB)
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(4 * TB + 2 * SB + VB) / 2];
  const uint32_t sm = lds_address(smem);
  const uint32_t vbase = sm + 4 * TB + 2 * SB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;

  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int bh = L / num_ktiles, kt = L % num_ktiles;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int k0 = kt * kBwdRows;
  const int key = k0 + wave * 32 + l32;
  const bool kv = key < N;
  TileCopy<D, BQ, kSwzKV> qcp;
  TileCopy<D, BQ, kSwzKV> dcp;
  qcp.init(wave, lane);
  dcp.init(wave, lane);
  LaneOffsets<D> lo;
  lo.init(lane, 0);
  // this wave's 32 V rows; kv_swz depends on the row modulo 16 only, so the
  // offsets of a 32-row tile serve them
  const uint32_t vwave = vbase + static_cast<uint32_t>(wave) * 32u * D * 2u;
  const float2* sh = stats + static_cast<size_t>(bh) * N;
  // the tile's 32 (lse2, -D) pairs, split on the way into LDS: lanes 0..31
  // copy the lse2 of rows 0..31, lanes 32..63 their -D, so the stage holds
  // an lse2 plane then a -D plane (128 bytes each)
  const uint32_t stats_voff = static_cast<uint32_t>(lane & 31) * 8u + static_cast<uint32_t>(hi) * 4u;
  auto stats_copy = [&](int q0, uint32_t dst) {
    if (wave == 0) {
      const int rows = N - q0 > 0 ? N - q0 : 0;
      const auto rsrc = buffer_rsrc(sh + q0, static_cast<uint32_t>(rows) * 8u);
      lds_dma4(rsrc, stats_voff, dst);
    }
  };
  const int NT = (N + BQ - 1) / BQ;
  {
    TileCopy<D, kBwdRows, kSwzKV> vcp;                   // the workgroup's 128 V rows, once
    vcp.init(wave, lane);
    vcp.copy(V + head, k0, N, vbase);
  }
  qcp.copy(Q + head, 0, N, sm);
  dcp.copy(dO + head, 0, N, sm + 2 * TB);
  stats_copy(0, sm + 4 * TB);

  vec8 kf[D / 16];
  load_row_frags<T, D>(kf, K + head + static_cast<size_t>(key) * D, kv, hi);
  const float c2 = scale * kLog2e;
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) dk[cb] = dv[cb] = f32x16{};

  auto tile = [&](auto par, int j) {
    constexpr int P = decltype(par)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);   // dropped again at the tile's end
    if (j + 1 < NT) {
      qcp.copy(Q + head, (j + 1) * BQ, N, sm + (1 - P) * TB);
      dcp.copy(dO + head, (j + 1) * BQ, N, sm + (3 - P) * TB);
      stats_copy((j + 1) * BQ, sm + 4 * TB + (1 - P) * SB);
    }
    const uint32_t qs = sm + P * TB, dos = sm + (2 + P) * TB, ss = sm + 4 * TB + P * SB;
    // this lane's 16 query rows: 8*g + 4*hi + 0..3 for g = 0..3, register
    // 4*g + i of both accumulators.  dP starts from -D of its row, so the
    // accumulator ends as dP - D and dS = P * (dP - D) takes one multiply.
    f32x16 s = f32x16{}, dp;
    u32x4 l2w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t a = ss + static_cast<uint32_t>(8 * g + 4 * hi) * 4u;
      l2w[g] = lds_read16(a);
      const u32x4 nd = lds_read16(a + 128u);
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[4 * g + i] = __uint_as_float(nd[i]);
    }
    rows_times<T, D>(s, qs, lo, kf);         // S  (queries x keys)
    rows_times_lds<T, D>(dp, dos, vwave, lo);  // dP - D
    const int qvalid = N - j * BQ;
    f32x16 p, dsv;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const int qi = 8 * g + 4 * hi + i;
        float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -__uint_as_float(l2w[g][i])));
        // Query rows at or beyond N need no mask: their Q and dO rows and
        // their statistics arrive as zeros, so P = 1 there meets dO = 0 in
        // dV and dS = 1 * (0 - 0) = 0 in dK -- exact zeros either way.  At
        // d = 128 dropping the select saves 16 VALU instructions per tile
        // (2% of the backward); at d = 64 the select-free instance measured
        // slower on short sequences, so it keeps the mask.
        if (D == 64) pr = qi < qvalid ? pr : 0.f;
        p[r] = pr;
        dsv[r] = pr * dp[r];
      }
    }
    vec8 pp[2], pd[2];
    pack_b<T>(p, pp);
    pack_b<T>(dsv, pd);
    cols_times<T, D>(dv, dos, lo, pp);       // dV^T += dO^T P
    cols_times<T, D>(dk, qs, lo, pd);        // dK^T += Q^T dS
    __builtin_amdgcn_s_setprio(0);
  };
  int j = 0;
  for (; j + 1 < NT; j += 2) {
    tile(P0{}, j);
    tile(P1{}, j + 1);
  }
  if (j < NT) tile(P0{}, j);
  if (kv) {
    store_rowmajor<T, D>(dK + head + static_cast<size_t>(key) * D, dk, hi, scale);
    store_rowmajor<T, D>(dV + head + static_cast<size_t>(key) * D, dv, hi, 1.f);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

template <class T, int D>
hipError_t launch_bwd_t(const BwdArgs& a) {
  const int64_t rows = a.BH * a.N;
  {
    constexpr int RPB = 256 / (D / 8);
    const int64_t wg = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_stats_kernel<T, D>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                       a.stream, static_cast<const uint16_t*>(a.O),
                       static_cast<const uint16_t*>(a.dO), a.LSE, static_cast<float2*>(a.stats),
                       rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tiles = static_cast<int>((a.N + kBwdRows - 1) / kBwdRows);
  const int64_t wg = a.BH * tiles;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                     a.stream, static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.dO),
                     static_cast<const float2*>(a.stats), static_cast<uint16_t*>(a.dQ),
                     static_cast<int>(a.N), tiles, static_cast<int>(wg), a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                     a.stream, static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.dO),
                     static_cast<const float2*>(a.stats), static_cast<uint16_t*>(a.dK),
                     static_cast<uint16_t*>(a.dV), static_cast<int>(a.N), tiles,
                     static_cast<int>(wg), a.scale);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_workgroups(int64_t BH, int64_t N) {
  return BH * ((N + kBwdRows - 1) / kBwdRows);
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.dtype == kDtypeBF16) return a.d == 128 ? launch_bwd_t<Bf16, 128>(a) : launch_bwd_t<Bf16, 64>(a);
  return a.d == 128 ? launch_bwd_t<F16, 128>(a) : launch_bwd_t<F16, 64>(a);
}

}  // namespace iofa
