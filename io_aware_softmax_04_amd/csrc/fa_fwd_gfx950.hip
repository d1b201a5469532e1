// Fused exact-attention forward for gfx950 (CDNA4).
//
// Method: xinc.fun archive 235, "6. 标准注意力为什么慢" (tiles of Q, K, V on
// chip, output accumulated directly, S and P never stored) and
// "7. Online Softmax" (running max m, denominator l and un-normalised output
// z per query row; a block of new scores rescales the old l and z by
// e^{m_old - m_new}; o = z / l at the end); ctyun.cn FlashAttention article,
// "核心思想" (blocks of the matrices staged in fast on-chip memory).
//
// gfx950 mapping (16-bit inputs):
//   * 8 waves per CU, two per SIMD: one workgroup of 8 waves = 256 query
//     rows of one head per CU at d = 128 when the grid still gives every CU
//     one, otherwise two workgroups of 4 waves = 128 rows each; each wave
//     owns 32 query rows for the whole key sweep and keeps their Q fragments
//     in VGPRs;
//   * the wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (fp32 acc): each
//     lane then holds one query column, so the row max and row sum are
//     in-lane over the tile's scores plus one exchange with the lane 32 apart
//     (v_permlane32_swap);
//   * O^T = V^T P^T takes P (rounded to the input type) straight from the
//     same registers as its B operand; V^T fragments come from the row-major
//     V tile through the transposing ds_read_b64_tr_b16;
//   * K and V tiles (32 keys at d = 128, 64 at d = 64) are copied global ->
//     LDS directly (buffer_load_dwordx4 ... lds, swizzled rows, range-checked
//     so rows past N arrive as zeros) into rings of four stages each: a K
//     tile three iterations ahead, a V tile one ahead;
//   * three-stage software pipeline: while the VALU computes the softmax of
//     tile j, the MFMA unit runs P_{j-1} V_{j-1} and the scores of tile j+1,
//     none of which depend on that softmax; one barrier per two tiles (the
//     four-stage rings keep a barrier between every copy and its reads, and
//     between every read and the copy that overwrites the stage); the score
//     and P V products alternate, and the wave runs them at raised issue
//     priority, dropped for the wait and barrier that close the tile;
//   * the loop is unrolled by four so every LDS stage offset is a constant:
//     each LDS read is a per-lane address computed once plus an immediate;
//   * exponentials are exp2 with log2(e) folded into the fp32 scale; the row
//     sum adds the fp32 exponentials, so the log-sum-exp keeps fp32 accuracy.
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace iofa {

// Waves per workgroup of the 16-bit kernel: 4 (two workgroups per CU) or 8
// (one).  With 8, all eight waves of a CU share the workgroup's barriers and
// so stay within two key tiles of each other: with two 4-wave workgroups per
// CU one of them ran ahead of the other (398 to 597 us for the same work at
// B1 H32 N16384), the workgroups of an XCD drifted apart by up to 3.4 MiB of
// K and V, and heads whose keys exceed the XCD's L2 were fetched 3.7 times
// instead of twice.  The launch takes 8 at d = 128 when that still gives
// every CU a workgroup (measured the same or faster there, B2 H8 N8191 2%
// faster), and 4 otherwise (at d = 64 8 measured 4% slower at B4 H16 N1024;
// a grid of fewer 8-wave workgroups than CUs would leave CUs idle).  Queries
// shorter than one 4-wave tile (decode) also take 4: the workgroup is then
// bound by its stream of keys and values, and the same number of 4-wave
// workgroups measured 12-23% faster there (B8 H32 Nq1 Nk8192 182 against
// 236 us).  Both forms do the same arithmetic per wave, so their results are
// identical.
template <int D, int BC, int NW_ = 4>
struct FusedCfg {
  static constexpr int NW = NW_;          // waves per workgroup
  static constexpr int BR = 32 * NW;      // query rows per workgroup
  static constexpr int SB = BC / 32;      // 32-key score blocks per tile
  static constexpr int KSTEPS = BC / 16;  // 16-key steps of P V per tile
  static constexpr int TILE = BC * D;     // elements of one K or V stage
  static constexpr uint32_t TB = TILE * 2u;   // bytes of one stage
  static constexpr int STAGES = 4;        // ring of LDS stages for K and for V
  static constexpr int SMEM = 2 * STAGES * TILE;   // K stages 0..3, then V stages 0..3
};

// The running maximum is only moved when a tile's maximum exceeds it by more
// than this many log2 units.  The result o = z / l and the log-sum-exp
// m + log2 l hold for any reference value m; keeping m within 8 of the true
// maximum bounds every exponential by 2^8, and the O accumulator is then
// rescaled only on the (rare, wave-uniform) tiles that move m.
constexpr float kRescaleSlack = 8.0f;
// Largest partial row sum (per lane, per tile) accepted without moving the
// reference maximum.  It bounds every unnormalised weight, which is rounded
// to the input type for the P V product: 2^32 for bf16 (range of fp32),
// 2^15 for fp16 (largest finite value 65504).
template <class T>
constexpr float kLazyBound = 4294967296.0f;
template <>
constexpr float kLazyBound<F16> = 32768.0f;

// One wave's share of the online-softmax recurrence.
template <class T, int D, int BC>
struct WaveState {
  using C = FusedCfg<D, BC>;
  using vec8 = typename T::vec8;
  vec8 qf[D / 16];               // Q fragments (B operand of S^T = K Q^T)
  f32x16 o[D / 32];              // O^T accumulator: lane owns one query column
  float m_run;                   // reference maximum, log2 units of scaled scores
  float l_run;                   // this lane half's share of the denominator (the
                                 // keys it holds), relative to m_run; the two
                                 // halves are added in the epilogue
  int hi;                        // lane half (0: lanes 0-31, 1: lanes 32-63)
  uint32_t k_addr[D / 16];       // LDS byte address of the K fragment, stage 0
  uint32_t v_addr[D / 32];       // LDS byte address of the V^T read, stage 0

  // smem_byte: LDS byte address of the stage area (K stage 0).
  __device__ inline void init_lanes(int lane, uint32_t smem_byte) {
    const int l32 = lane & 31;
    hi = lane >> 5;
    // K: lane (l32, hi) reads key row l32 (+32 per score block), columns
    // 16*kk + 8*hi .. +7, i.e. chunk 2*kk + hi, stored at chunk
    // (2*kk + hi) ^ k_swz(row); the swizzle is the same for row + 32.
    const int kswz = k_swz<D>(l32);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      k_addr[kk] = smem_byte + static_cast<uint32_t>(l32 * D + (((2 * kk + hi) ^ kswz) * 8)) * 2u;
    // V: ds_read_b64_tr_b16: in each 16-lane group, lane t supplies row
    // key0 + t/4, columns c0 + 4*(t%4) .. +3 and receives column c0 + t of
    // rows key0 .. key0+3.  Group g = lane/16 covers lane half g/2 (keys
    // 4*(g/2) + ...) and column half g%2.  The swizzle depends on row % 4,
    // the same for every key step.
    const int g = lane >> 4, t = lane & 15;
    const int row = 4 * (g >> 1) + (t >> 2);
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int col = 32 * cb + 16 * (g & 1) + 4 * (t & 3);
      const int chunk = (col >> 3) ^ v_swz<D>(row);
      v_addr[cb] = smem_byte + C::STAGES * C::TB + static_cast<uint32_t>(row * D + chunk * 8 + (col & 7)) * 2u;
    }
  }

  // a3: scores S^T of one tile (raw dot products) from K stage S.
  template <int S>
  __device__ inline void scores(f32x16 (&s)[C::SB]) const {
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) s[sb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) {
        const auto a = __builtin_bit_cast(vec8, lds_read16(k_addr[kk] + S * C::TB + 32 * sb * D * 2));
        s[sb] = T::mfma(a, qf[kk], s[sb]);
      }
    }
  }

  // a6: acc += P V for one tile from V stage S.  The A operand (V^T) comes
  // from two transposed reads: keys 16*ks + 4*hi + 0..3 and
  // 16*ks + 8 + 4*hi + 0..3, the keys the P registers hold in k-slots
  // 8*hi + 0..3 and 8*hi + 4..7.
  template <int S>
  __device__ inline void pv(const vec8 (&pk)[C::KSTEPS]) {
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const uint32_t a0 = v_addr[cb] + S * C::TB + 16 * ks * D * 2;
        const s16x4 lo = lds_read_tr8(a0);
        const s16x4 up = lds_read_tr8(a0 + 8 * D * 2);
        const auto a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        o[cb] = T::mfma(a, pk[ks], o[cb]);
      }
    }
  }

  // a6 of the previous tile and a3 of the next, their products alternating
  // (score product i, then P V product i) so each K fragment read has
  // several products of lead time instead of one.
  template <int SV, int SK>
  __device__ inline void pv_scores(const vec8 (&pk)[C::KSTEPS], f32x16 (&s)[C::SB]) {
    constexpr int NS = (D / 16) * C::SB;
    constexpr int NP = C::KSTEPS * (D / 32);
    constexpr int NI = NS > NP ? NS : NP;
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) s[sb] = f32x16{};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i < NS) {
        const int kk = i / C::SB, sb = i % C::SB;
        const auto a = __builtin_bit_cast(vec8, lds_read16(k_addr[kk] + SK * C::TB + 32 * sb * D * 2));
        s[sb] = T::mfma(a, qf[kk], s[sb]);
      }
      if (i < NP) {
        const int ks = i / (D / 32), cb = i % (D / 32);
        const uint32_t a0 = v_addr[cb] + SV * C::TB + 16 * ks * D * 2;
        const s16x4 lo = lds_read_tr8(a0);
        const s16x4 up = lds_read_tr8(a0 + 8 * D * 2);
        const auto a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        o[cb] = T::mfma(a, pk[ks], o[cb]);
      }
    }
  }

  // a4 + a5: tile maximum, reference-maximum update, exponentials, row sum,
  // packing of P to the input type.  Returns the rescale factor of the older
  // terms.  TAIL masks keys at or beyond keys_valid to weight 0.
  template <bool TAIL>
  __device__ inline float softmax(f32x16 (&s)[C::SB], vec8 (&pk)[C::KSTEPS], float c2,
                                  int keys_valid) {
    float mraw = -__builtin_inff();
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (TAIL) {
          const int key = 32 * sb + 8 * (r >> 2) + 4 * hi + (r & 3);
          mraw = (key < keys_valid) ? fmaxf(mraw, s[sb][r]) : mraw;
        } else {
          mraw = fmaxf(mraw, s[sb][r]);
        }
      }
    mraw = halfwave_max(mraw);
    const float mt = mraw * c2;          // this tile's maximum, log2 units (c2 >= 0)
    const bool move = mt > m_run + kRescaleSlack;   // always on the first tile
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
    m_run = move ? mt : m_run;
    const float msub = m_run;
    float rs = 0.f;
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[sb][r], c2, -msub));
        if (TAIL) {
          const int key = 32 * sb + 8 * (r >> 2) + 4 * hi + (r & 3);
          p = (key < keys_valid) ? p : 0.f;
        }
        s[sb][r] = p;
        rs += p;
      }
    }
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const f32x16& p = s[ks >> 1];
      const int b = 8 * (ks & 1);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = T::pack(p[b + 2 * e], p[b + 2 * e + 1]);
      pk[ks] = __builtin_bit_cast(vec8, w);
    }
    l_run = alpha * l_run + rs;
    return alpha;
  }

  // a5 without a4 (the usual case after the first tile): exponentials
  // against the current reference maximum, packing, and this lane's partial
  // row sum, which is returned.  s is left intact.  Every exponential is at
  // most the partial sum, so when the sum is at most kLazyBound on all lanes
  // (commit_lazy), every term fits the packed type, the accumulators stay far
  // from overflow, and the reference need not move; otherwise (a score above
  // the reference by more than log2 kLazyBound, or the -inf reference of an
  // empty state) the tile is redone with its maximum by softmax<false>.  A
  // failed check implies a tile maximum more than kRescaleSlack above the
  // reference (at most 32 terms of 2^kRescaleSlack per lane stay below both
  // bounds), so the redo always moves the reference.
  __device__ inline float softmax_lazy(const f32x16 (&s)[C::SB], vec8 (&pk)[C::KSTEPS],
                                       float c2) const {
    const float msub = m_run;
    float rs = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const f32x16& v = s[ks >> 1];
      const int b = 8 * (ks & 1);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(v[b + 2 * e], c2, -msub));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(v[b + 2 * e + 1], c2, -msub));
        // the sum starts from its first term, saving the add of 0 the compiler
        // must keep (0 + x is not x for x = -0); measured 0.9% faster at
        // d = 128 and no faster at d = 64, where the first form stays
        rs = (D == 128 && ks == 0 && e == 0) ? p0 : rs + p0;
        rs += p1;
        w[e] = T::pack(p0, p1);
      }
      pk[ks] = __builtin_bit_cast(vec8, w);
    }
    return rs;
  }
  // Accept a lazy tile (returns false) or redo it with its maximum (returns
  // true, with the rescale factor of the older terms in alpha).
  __device__ inline bool commit_lazy(float rs, f32x16 (&s)[C::SB], vec8 (&pk)[C::KSTEPS],
                                     float c2, float& alpha) {
    if (__all(rs <= kLazyBound<T>)) {
      l_run += rs;
      return false;
    }
    vec8 lazy[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) lazy[ks] = pk[ks];
    alpha = softmax<false>(s, pk, c2, BC);
    if constexpr (D == 128) {
      // A lane whose reference did not move (alpha == 1) recomputed exactly
      // the lazy weights, so it may keep them.  Reading them here gives the
      // lazy packing a use on this path too: the compiler then packs ahead
      // of the branch, inside the interleave, instead of holding the sixteen
      // fp32 weights across all the products (with the reads kept ahead,
      // 1.1-1.4% faster at d = 128, bit-identical; d = 64 measured slower)
      const bool moved = alpha != 1.f;
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) pk[ks] = moved ? pk[ks] : lazy[ks];
    }
    return true;
  }

  __device__ inline void rescale(float alpha) {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) o[cb] *= alpha;
    }
  }
};

// Per wave, tile t of the key sweep (NT tiles) is processed in three steps:
// its scores in iteration t-1, its softmax in iteration t, its P V product
// in iteration t+1.  K tile t lives in K stage t%4, copied in iteration t-3;
// V tile t in V stage t%4, copied in iteration t-1.  Iteration j (P = j%4):
//   top     direct copies K_{j+3} -> K stage (j+3)%4 (last read in iteration
//           j-2) and V_{j+1} -> V stage (j+1)%4 (last read in iteration j-2);
//   middle  softmax_j (VALU) interleaved with P_{j-1} V_{j-1} (V stage
//           (j-1)%4) and scores_{j+1} (K stage (j+1)%4) on the MFMA unit;
//   bottom  rescale of O if the reference maximum moved; after odd j only:
//           wait for the copies in flight, barrier.
// Barriers after every odd iteration (and after iteration 0) put one between
// each copy and its first read (a K copy in j and its read in j+2, a V copy
// in j and its read in j+2) and between each last read and the overwriting
// copy (read in j-2, copy in j); one barrier per tile measured 2.2-2.7%
// slower at B2 H16 N4096, B2 H8 N8191 and B1 H32 N16384, bit-identical.
//
// Q and O hold Nq rows per head, K and V Nk (the same except for attention
// of one sequence of queries over another of keys, decode included).
// With PARTIAL the workgroup covers only the keys of its split (key_range)
// and writes the normalised partial output in fp32 to Out[(split*BH + bh),
// q, :] and its log-sum-exp to Lse[(split*BH + bh), q]; the partials are
// combined by fa_merge_kernel.  Otherwise (one split) it writes O in the
// input type and the final LSE.  STREAM (fa_fwd_16_stream_kernel below)
// marks the K and V copies non-temporal and changes the schedule above: V
// copied in iteration t-2, a wait and barrier after every iteration that
// leaves the three newest tile copies in flight, and a full wait only in the
// last iteration.
template <class T, int D, int BC, bool PARTIAL, int NW, bool STREAM>
__device__ __forceinline__ void fused16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, void* __restrict__ Out,
    float* __restrict__ Lse, int Nq, int Nk, int BH, int num_qtiles, int num_splits, int num_wg,
    float scale) {
  using C = FusedCfg<D, BC, NW>;
  using vec8 = typename T::vec8;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::SMEM];
  const uint32_t sm = lds_address(smem);
  const uint32_t kst[4] = {sm, sm + C::TB, sm + 2 * C::TB, sm + 3 * C::TB};
  const uint32_t vst[4] = {sm + 4 * C::TB, sm + 5 * C::TB, sm + 6 * C::TB, sm + 7 * C::TB};

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  const GridPos gp = grid_pos(num_qtiles, num_splits, num_wg);
  const int bh = gp.bh, qt = gp.qt;
  const int2 kr = key_range(Nk, BC, gp.split, num_splits);
  const int NK = kr.y;                 // keys of this workgroup
  const size_t head = static_cast<size_t>(bh) * Nq * D;    // Q and O rows of this head
  const size_t khead = static_cast<size_t>(bh) * Nk * D;   // K and V rows of this head
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + khead + static_cast<size_t>(kr.x) * D;
  const uint16_t* Vh = V + khead + static_cast<size_t>(kr.x) * D;

  const int NT = (NK + BC - 1) / BC;   // key tiles
  const bool ragged = (NK % BC) != 0;
  TileCopy<D, BC, kSwzK, C::NW, STREAM> kcp;
  TileCopy<D, BC, kSwzV, C::NW, STREAM> vcp;
  kcp.init(wave, lane);
  vcp.init(wave, lane);

  // K is copied 3 tiles ahead of its scores, V VA tiles ahead of its P V
  // product.  The tile kernel waits for every copy at each barrier (after odd
  // iterations); the stream form (short query blocks, bound by the stream of
  // K and V) synchronises after every iteration and keeps its newest KEEP
  // tile copies in flight across each wait, V being copied two ahead so the
  // ring still has the stage (a host model of both schedules checks every
  // stage's copy, wait, barrier and read order).
  constexpr int VA = STREAM ? 2 : 1;
  constexpr int KEEP = STREAM ? 3 : 0;
  auto wait_copies = [&](auto keep_c) {
    constexpr int n = decltype(keep_c)::value * decltype(kcp)::PER_WAVE;   // instructions
    static_assert(n < 64, "vmcnt holds 6 bits");
    // vmcnt(n) (bits 3:0 and 15:14), expcnt(7), lgkmcnt(0): the LDS reads
    // are done as well
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
  };
  using Keep0 = std::integral_constant<int, 0>;
  using KeepN = std::integral_constant<int, KEEP>;

  // a2 prologue: K_0, K_1, K_2 and V_0 (.. V_{VA-1}) in flight while Q is
  // loaded
  kcp.copy(Kh, 0, NK, kst[0]);
  kcp.copy(Kh, BC, NK, kst[1]);
  kcp.copy(Kh, 2 * BC, NK, kst[2]);
  vcp.copy(Vh, 0, NK, vst[0]);
  if constexpr (VA == 2) vcp.copy(Vh, BC, NK, vst[1]);

  // a1: this lane's query row, its Q fragments, the running state.  A
  // negative scale is folded into Q (negation is exact) so the scale applied
  // to the fp32 scores is c2 = |scale| * log2(e) >= 0.
  WaveState<T, D, BC> ws;
  ws.init_lanes(lane, sm);
  const int q = qt * C::BR + wave * 32 + (lane & 31);
  const uint32_t flip = scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (q < Nq) w = *reinterpret_cast<const u32x4*>(Qh + static_cast<size_t>(q) * D + 16 * kk + 8 * ws.hi);
    w ^= flip;
    ws.qf[kk] = __builtin_bit_cast(vec8, w);
  }
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) ws.o[cb] = f32x16{};
  ws.m_run = -__builtin_inff();
  ws.l_run = 0.f;
  const float c2 = fabsf(scale) * kLog2e;

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa[C::SB], sb[C::SB];
  vec8 pa[C::KSTEPS], pb[C::KSTEPS];
  // A wave whose 32 query rows all lie past the last query row (a query
  // block shorter than the workgroup's, one decode row per head above all)
  // computes nothing: it issues its share of every K and V copy and joins
  // every wait and barrier in the same order as the computing waves, which
  // run the same program below with IDLE false.
  const bool idle_wave = qt * C::BR + wave * 32 >= Nq;   // wave-uniform
  auto body = [&](auto idle_c) {
    constexpr bool IDLE = decltype(idle_c)::value;
    if constexpr (!IDLE) ws.template scores<0>(sa);

    constexpr int NM = 2 * (D / 16) * C::SB;          // products per iteration
    constexpr int NRD = (D / 16) * C::SB + 2 * NM / 2;  // K reads + 2 per P V product
    // LDS reads issued ahead of the interleaved products: at d = 128 kept 4
    // ahead for the whole tile (1.1-1.4% faster at B2 H16 N4096 and B2 H8
    // N8191 than 6 ahead with the lead draining over the tile); 8 at d = 64
    constexpr int LEAD = D == 128 ? 4 : 8;
    // keep_c: tile copies left in flight by the wait (0 in the last iteration)
    auto bottom = [&](float alpha, auto keep_c) {
      if constexpr (!IDLE) ws.rescale(alpha);
      if constexpr (decltype(keep_c)::value == 0)
        __builtin_amdgcn_s_waitcnt(0);
      else
        wait_copies(keep_c);
      __syncthreads();
    };
    // one full iteration j with parity P (compile-time)
    auto iteration = [&](auto par, int j, f32x16 (&s_cur)[C::SB], f32x16 (&s_nxt)[C::SB],
                         vec8 (&p_prev)[C::KSTEPS], vec8 (&p_cur)[C::KSTEPS]) {
      constexpr int P = decltype(par)::value;   // j % 4
      if constexpr (IDLE) {
        kcp.copy(Kh, (j + 3) * BC, NK, kst[(P + 3) % 4]);
        vcp.copy(Vh, (j + VA) * BC, NK, vst[(P + VA) % 4]);
      } else {
        // raised issue priority from the copies through the products; dropped
        // again before the wait and barrier (measured 0.8% faster at d = 128,
        // 3.8% at d = 64, bit-identical output)
        __builtin_amdgcn_s_setprio(1);
        kcp.copy(Kh, (j + 3) * BC, NK, kst[(P + 3) % 4]);
        vcp.copy(Vh, (j + VA) * BC, NK, vst[(P + VA) % 4]);
        const float rs = ws.softmax_lazy(s_cur, p_cur, c2);
        ws.template pv_scores<(P + 3) % 4, (P + 1) % 4>(p_prev, s_nxt);
        // d = 128 keeps its reads LEAD ahead for the whole tile, with three
        // vector instructions per product (four: 1.1-1.5% slower at B2 H16
        // N4096, B2 H8 N8191 and B1 H32 N16384; two: 0.5% slower); at d = 64 the
        // draining order with four measured faster (21.0 vs 21.7 us at
        // B4 H16 N1024)
        if constexpr (D == 128)
          interleave_mfma_valu_lead<NM, NRD, LEAD, 3>();
        else
          interleave_mfma_valu<NM, NRD, LEAD, 4>();
        // the redo decision is wave-uniform, so the accepted path (almost every
        // tile) carries no rescale factor and no rescale test
        float alpha;
        if (ws.commit_lazy(rs, s_cur, p_cur, c2, alpha)) ws.rescale(alpha);
        __builtin_amdgcn_s_setprio(0);
      }
      if constexpr (STREAM) {
        wait_copies(KeepN{});
        __syncthreads();
      } else if constexpr (P % 2 == 1) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    };
    // the last iteration j = NT-1 (parity P): no scores, maybe a ragged tile
    auto last = [&](auto par, int j, f32x16 (&s_cur)[C::SB], vec8 (&p_prev)[C::KSTEPS],
                    vec8 (&p_cur)[C::KSTEPS]) {
      constexpr int P = decltype(par)::value;   // j % 4
      if constexpr (IDLE) {
        bottom(0.f, Keep0{});
      } else {
        const float alpha = ragged ? ws.template softmax<true>(s_cur, p_cur, c2, NK - j * BC)
                                   : ws.template softmax<false>(s_cur, p_cur, c2, BC);
        if (j > 0) ws.template pv<(P + 3) % 4>(p_prev);
        bottom(alpha, Keep0{});
        ws.template pv<P>(p_cur);
      }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;

    if (NT == 1) {
      last(P0{}, 0, sa, pb, pa);
    } else {
      // iteration 0: softmax_0 with scores_1
      kcp.copy(Kh, 3 * BC, NK, kst[3]);
      vcp.copy(Vh, VA * BC, NK, vst[VA]);
      if constexpr (IDLE) {
        bottom(0.f, KeepN{});
      } else {
        const float alpha = ws.template softmax<false>(sa, pa, c2, BC);
        ws.template scores<1>(sb);
        constexpr int NS1 = (D / 16) * C::SB;
        interleave_mfma_valu<NS1, NS1, 2, 4>();
        bottom(alpha, KeepN{});
      }
      // iterations 1 .. NT-2, four per trip so register sets alternate and
      // every stage index is a constant
      int j = 1;
      for (; j + 3 < NT - 1; j += 4) {
        iteration(P1{}, j, sb, sa, pa, pb);
        iteration(P2{}, j + 1, sa, sb, pb, pa);
        iteration(P3{}, j + 2, sb, sa, pa, pb);
        iteration(P0{}, j + 3, sa, sb, pb, pa);
      }
      if (j < NT - 1) {
        iteration(P1{}, j, sb, sa, pa, pb);
        if (j + 1 < NT - 1) {
          iteration(P2{}, j + 1, sa, sb, pb, pa);
          if (j + 2 < NT - 1) {
            iteration(P3{}, j + 2, sb, sa, pa, pb);
            last(P0{}, j + 3, sa, pb, pa);
          } else {
            last(P3{}, j + 2, sb, pa, pb);
          }
        } else {
          last(P2{}, j + 1, sa, pb, pa);
        }
      } else {
        last(P1{}, j, sb, pa, pb);
      }
    }
  };
  if (idle_wave)
    body(std::true_type{});
  else
    body(std::false_type{});

  // a7: O = acc / l rounded to the input type (or kept fp32 for a partial);
  // LSE = ln2 * (m + log2 l).  Lane half hi holds columns 32*cb + 8*g + 4*hi
  // + 0..3 in registers 4*g .. 4*g+3.
  if (q < Nq) {
    const float l = halfwave_sum(ws.l_run);
    const float inv_l = 1.0f / l;
    const float lse = (ws.m_run + __builtin_amdgcn_logf(l)) * kLn2;
    if constexpr (PARTIAL) {
      const size_t row = (static_cast<size_t>(gp.split) * BH + bh) * Nq + q;
      float* Oq = static_cast<float*>(Out) + row * D;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(Oq + 32 * cb + 8 * g + 4 * ws.hi) =
              make_float4(ws.o[cb][4 * g + 0] * inv_l, ws.o[cb][4 * g + 1] * inv_l,
                          ws.o[cb][4 * g + 2] * inv_l, ws.o[cb][4 * g + 3] * inv_l);
      if (ws.hi == 0) Lse[row] = lse;
    } else {
      uint16_t* Oq = static_cast<uint16_t*>(Out) + head + static_cast<size_t>(q) * D;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = T::pack(ws.o[cb][4 * g + 0] * inv_l, ws.o[cb][4 * g + 1] * inv_l);
          w[1] = T::pack(ws.o[cb][4 * g + 2] * inv_l, ws.o[cb][4 * g + 3] * inv_l);
          *reinterpret_cast<u32x2*>(Oq + 32 * cb + 8 * g + 4 * ws.hi) = w;
        }
      }
      if (ws.hi == 0) Lse[static_cast<size_t>(bh) * Nq + q] = lse;
    }
  }
}

template <class T, int D, int BC, bool PARTIAL, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fa_fwd_16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, void* __restrict__ Out,
    float* __restrict__ Lse, int Nq, int Nk, int BH, int num_qtiles, int num_splits, int num_wg,
    float scale) {
  fused16<T, D, BC, PARTIAL, NW, false>(Q, K, V, Out, Lse, Nq, Nk, BH, num_qtiles, num_splits,
                                        num_wg, scale);
}

// Queries shorter than one 4-wave tile (decode): each (head, key range) has
// a single workgroup, so every K and V byte is read by one workgroup only
// and the workgroup is bound by that stream.  The copies are marked
// non-temporal (with K and V read from HBM, B8 H32 Nq1 Nk8192: 161 against
// 182 us; the same marking in the kernel above, whose K and V tiles other
// query tiles read again from L2, measured up to 1.6% slower at B1 H32
// N16384), and the schedule keeps three tile copies in flight across its
// barriers instead of draining them every two tiles (153 against 161 us;
// B2 H16 Nq1 Nk4096: 16.0 against 18.0 us with the merge).
template <class T, int D, int BC, bool PARTIAL>
__global__ __launch_bounds__(256, 2) void fa_fwd_16_stream_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, void* __restrict__ Out,
    float* __restrict__ Lse, int Nq, int Nk, int BH, int num_qtiles, int num_splits, int num_wg,
    float scale) {
  fused16<T, D, BC, PARTIAL, 4, true>(Q, K, V, Out, Lse, Nq, Nk, BH, num_qtiles, num_splits,
                                      num_wg, scale);
}

// ---------------------------------------------------------------- fp32 path
//
// fp32 inputs keep every product and sum in fp32 on the vector ALUs (on
// MI355X the fp32 matrix and vector peaks are equal).  Workgroup = 32 query
// rows x 8 threads per row; each thread owns D/8 columns of q and of the
// output accumulator; a score is the 8-lane sum of partial dot products.
// K and V tiles of 32 keys are staged in LDS.

// With PARTIAL: keys of the workgroup's split only, output rows
// (split*BH + bh, q) of the fp32 partials (see fa_fwd_16_kernel).
template <int D, bool PARTIAL>
__global__ __launch_bounds__(256) void fa_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
    int Nq, int Nk, int BH, int num_qtiles, int num_splits, int num_wg, float scale) {
  constexpr int QPB = 32, TPQ = 8, DPT = D / TPQ, BC = 32, LS = D + 4;
  __shared__ __attribute__((aligned(16))) float Ks[BC * LS];
  __shared__ __attribute__((aligned(16))) float Vs[BC * LS];

  const int tid = threadIdx.x;
  const GridPos gp = grid_pos(num_qtiles, num_splits, num_wg);
  const int bh = gp.bh, qt = gp.qt;
  const int2 kr = key_range(Nk, BC, gp.split, num_splits);
  const int kbeg = kr.x, kend = kr.x + kr.y;
  const size_t head = static_cast<size_t>(bh) * Nq * D;    // Q and O rows of this head
  const size_t khead = static_cast<size_t>(bh) * Nk * D;   // K and V rows of this head
  const int qi = tid / TPQ, part = tid % TPQ;
  const int q = qt * QPB + qi;
  const int c0 = part * DPT;

  float qv[DPT], ov[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    qv[e] = (q < Nq) ? Q[head + static_cast<size_t>(q) * D + c0 + e] : 0.f;
    ov[e] = 0.f;
  }
  float m_run = -__builtin_inff(), l_run = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += BC) {
    for (int i = tid; i < BC * D / 4; i += 256) {
      const int row = i / (D / 4), c4 = i % (D / 4);
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (k0 + row < kend) {
        kv = *reinterpret_cast<const float4*>(K + khead + static_cast<size_t>(k0 + row) * D + 4 * c4);
        vv = *reinterpret_cast<const float4*>(V + khead + static_cast<size_t>(k0 + row) * D + 4 * c4);
      }
      *reinterpret_cast<float4*>(Ks + row * LS + 4 * c4) = kv;
      *reinterpret_cast<float4*>(Vs + row * LS + 4 * c4) = vv;
    }
    __syncthreads();

    float sc[BC];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float part_dot = 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) part_dot = fmaf(qv[e], Ks[j * LS + c0 + e], part_dot);
      part_dot += __shfl_xor(part_dot, 1, TPQ);
      part_dot += __shfl_xor(part_dot, 2, TPQ);
      part_dot += __shfl_xor(part_dot, 4, TPQ);
      sc[j] = (k0 + j < kend) ? part_dot * scale : -__builtin_inff();
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = expf(m_run - msub);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      sc[j] = expf(sc[j] - msub);
      rs += sc[j];
    }
    l_run = alpha * l_run + rs;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      float acc = ov[e] * alpha;
#pragma unroll
      for (int j = 0; j < BC; ++j) acc = fmaf(sc[j], Vs[j * LS + c0 + e], acc);
      ov[e] = acc;
    }
    __syncthreads();
  }

  if (q < Nq) {
    const size_t row = PARTIAL ? (static_cast<size_t>(gp.split) * BH + bh) * Nq + q
                               : static_cast<size_t>(bh) * Nq + q;
#pragma unroll
    for (int e = 0; e < DPT; ++e) O[row * D + c0 + e] = ov[e] / l_run;
    if (part == 0) LSE[row] = m_run + logf(l_run);
  }
}

// ------------------------------------------------------------- launchers

// Keys per tile: 32 at d = 128 (keeps the three-stage pipeline's registers
// within the 256 a wave has at two waves per SIMD), 64 at d = 64.
template <int D>
constexpr int kFusedBC = D == 128 ? 32 : 64;

int fused_key_tile(int dtype, int64_t d) {
  if (dtype == kDtypeF32) return 32;
  return d == 128 ? kFusedBC<128> : kFusedBC<64>;
}

// Query rows per workgroup of the form with the most workgroups (the grid
// limit check) and waves of a launch (the split-KV heuristic).
int64_t fused_query_tile(int dtype) { return dtype == kDtypeF32 ? 32 : FusedCfg<128, 32>::BR; }

int64_t fused_waves(int dtype, int64_t BH, int64_t N, int64_t splits) {
  const int64_t br = fused_query_tile(dtype);
  return BH * splits * ((N + br - 1) / br) * 4;
}

// CUs of the current device (256 if it cannot be found out).
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <class T, int D, bool PARTIAL, int BC, int NW>
static hipError_t launch16_nw(const FwdArgs& a, int splits, void* out, float* lse) {
  using C = FusedCfg<D, BC, NW>;
  const int qtiles = static_cast<int>((a.N + C::BR - 1) / C::BR);
  const int64_t wg = a.BH * splits * qtiles;
  hipLaunchKernelGGL((fa_fwd_16_kernel<T, D, BC, PARTIAL, NW>), dim3(static_cast<unsigned>(wg)),
                     dim3(64 * NW), 0, a.stream, static_cast<const uint16_t*>(a.Q),
                     static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.V), out, lse,
                     static_cast<int>(a.N), static_cast<int>(a.Nk), static_cast<int>(a.BH), qtiles, splits,
                     static_cast<int>(wg), a.scale);
  return hipGetLastError();
}

template <class T, int D, bool PARTIAL, int BC = kFusedBC<D>>
static hipError_t launch16(const FwdArgs& a, int splits, void* out, float* lse) {
  constexpr int64_t BR4 = FusedCfg<D, BC, 4>::BR;
  if (a.N < BR4) {
    const int64_t wg = a.BH * splits;   // one query tile per head and split
    hipLaunchKernelGGL((fa_fwd_16_stream_kernel<T, D, BC, PARTIAL>), dim3(static_cast<unsigned>(wg)),
                       dim3(256), 0, a.stream, static_cast<const uint16_t*>(a.Q),
                       static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.V), out, lse,
                       static_cast<int>(a.N), static_cast<int>(a.Nk), static_cast<int>(a.BH), 1,
                       splits, static_cast<int>(wg), a.scale);
    return hipGetLastError();
  }
  if constexpr (D == 128) {
    constexpr int64_t BR8 = FusedCfg<D, BC, 8>::BR;
    if (a.BH * splits * ((a.N + BR8 - 1) / BR8) >= device_cus())
      return launch16_nw<T, D, PARTIAL, BC, 8>(a, splits, out, lse);
  }
  return launch16_nw<T, D, PARTIAL, BC, 4>(a, splits, out, lse);
}

template <int D, bool PARTIAL>
static hipError_t launch32(const FwdArgs& a, int splits, float* out, float* lse) {
  const int qtiles = static_cast<int>((a.N + 31) / 32);
  const int64_t wg = a.BH * splits * qtiles;
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, PARTIAL>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                     a.stream, static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                     static_cast<const float*>(a.V), out, lse, static_cast<int>(a.N),
                     static_cast<int>(a.Nk), static_cast<int>(a.BH), qtiles, splits,
                     static_cast<int>(wg), a.scale);
  return hipGetLastError();
}

template <bool PARTIAL>
static hipError_t launch_any(const FwdArgs& a, int splits, void* out, float* lse) {
  if (a.dtype == kDtypeBF16)
    return a.d == 128 ? launch16<Bf16, 128, PARTIAL>(a, splits, out, lse)
                      : launch16<Bf16, 64, PARTIAL>(a, splits, out, lse);
  if (a.dtype == kDtypeF16)
    return a.d == 128 ? launch16<F16, 128, PARTIAL>(a, splits, out, lse)
                      : launch16<F16, 64, PARTIAL>(a, splits, out, lse);
  float* o = static_cast<float*>(out);
  return a.d == 128 ? launch32<128, PARTIAL>(a, splits, o, lse)
                    : launch32<64, PARTIAL>(a, splits, o, lse);
}

int64_t fused_workgroups(int dtype, int64_t BH, int64_t N, int64_t splits) {
  const int64_t br = fused_query_tile(dtype);
  return BH * splits * ((N + br - 1) / br);
}

hipError_t launch_fused(const FwdArgs& a) { return launch_any<false>(a, 1, a.O, a.LSE); }

hipError_t launch_fused_partial(const FwdArgs& a, int splits, float* O_part, float* LSE_part) {
  return launch_any<true>(a, splits, O_part, LSE_part);
}

}  // namespace iofa
