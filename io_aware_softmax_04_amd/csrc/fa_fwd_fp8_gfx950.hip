// Fused exact-attention forward with FP8 inputs (OCP E4M3) for gfx950.
//
// Method: the online-softmax recurrence of the 16-bit fused forward
// (xinc.fun archive 235, "7. Online Softmax"; ctyun.cn FlashAttention
// article, "核心思想"), with the mixed-precision split of the same xinc page,
// "4. 减少访存的几种办法": the two matrix products take 8-bit floating-point
// operands, while accumulation, the softmax and the final normalisation stay
// in fp32.
//
// Values: Q, K, V hold E4M3 codes and each tensor has one fp32 scale; an
// element's value is its code's value times that scale (sq, sk, sv).  The
// scores are scale * sq * sk * (Q8 K8^T), accumulated in fp32 by
// v_mfma_f32_32x32x64_f8f6f4.  For the second product the weights are
// rounded to E4M3: each weight is formed as p8 = 8 * 2^(s - m) against a
// reference maximum m (the factor 8 keeps weights down to 2^-9 of the
// maximum inside E4M3's normal range), and a tile is accepted against the
// old reference only while every lane's partial sum of p8 is at most 448,
// the largest finite E4M3 value, which bounds each p8 by it; otherwise the
// tile is redone against its own maximum (then p8 <= 8).  The row sum adds
// the fp32 weights, so the log-sum-exp keeps fp32 accuracy.  O = sv * acc / l
// is written in bf16, LSE in fp32 (natural log, units of scaled scores).
//
// gfx950 mapping: workgroup = 4 waves x 32 query rows of one head, two
// workgroups per CU; tiles of 64 keys; per wave and tile S^T = K Q^T takes
// 2 x D/64 products of 32x32x64 (lane = query column, as in the 16-bit
// kernel) and O^T += V^T P^T takes D/32 products whose B operand is P packed
// straight from the score registers; the A operand V^T comes from the
// row-major V tile through ds_read_b64_tr_b8.  K and V tiles are copied
// global -> LDS by buffer_load ... lds into two stages each, and the loop
// runs the same three-stage pipeline as the 16-bit kernel: softmax of tile j
// on the VALU while the MFMA unit runs P_{j-1} V_{j-1} and the scores of
// tile j+1.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace iofa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct Fp8Cfg {
  static constexpr int NW = 4;             // waves per workgroup
  static constexpr int BR = 32 * NW;       // query rows per workgroup
  static constexpr int BC = 64;            // keys per tile
  static constexpr uint32_t TB = BC * D;   // bytes of one K or V stage
  static constexpr int KB = D / 64;        // 64-deep steps of a score product
  static constexpr int CB = D / 32;        // 32-row blocks of O^T
};

// p8 = 2^(s - m + kP8Shift); kP8Bound = largest finite E4M3 value.
constexpr float kP8Shift = 3.0f;
constexpr float kP8Bound = 448.0f;

// Both operands E4M3 (format selectors 0); scale operands 0 select the
// unscaled product.
__device__ inline f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS tile layouts (rows of D bytes, row-major, 16-byte chunks permuted
// within a row so that the reads below hit distinct banks):
//   K, read as 32-byte row fragments (two 16-byte reads, 16 consecutive rows
//   per 16-lane group): chunk c of row r sits at
//       c ^ ((r >> 1) & 7)   (D = 128)       c ^ ((r >> 2) & 3)   (D = 64)
//   V, read with ds_read_b64_tr_b8 (8 rows x 32 bytes per half-wave): the
//   pair of chunks p = c / 2 of row r sits at pair
//       p ^ ((((r >> 3) & 1) << 1) | ((r >> 1) & 1))   (D = 128)
//       p ^ ((r >> 3) & 1)                              (D = 64)
// Both depend on r mod 16 only.
template <int D>
__device__ inline int k8_swz(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D>
__device__ inline int v8_swz(int r) {
  return D == 128 ? (((((r >> 3) & 1) << 1) | ((r >> 1) & 1)) << 1) : (((r >> 3) & 1) << 1);
}

// Direct global -> LDS copy of one 64-row tile (rows of D bytes) by the 4
// waves of a workgroup: wave w writes the 1 KiB blocks w + 4i; every row a
// lane copies has the same swizzle (rows 16k apart).  Rows at or beyond N
// arrive as zeros (range-checked buffer).
template <int D, bool IS_V>
struct Fp8TileCopy {
  static constexpr int CH = D / 16;               // 16-byte chunks per row
  static constexpr int ROWS_PER_BLK = 64 / CH;    // rows in one 1 KiB block
  static constexpr int BLKS = Fp8Cfg<D>::TB / 1024;
  static constexpr int PER_WAVE = BLKS / 4;
  static constexpr int ROW_STEP = 4 * ROWS_PER_BLK;
  static_assert(PER_WAVE * 4 == BLKS, "tile must split over the waves");
  static_assert(ROW_STEP % 16 == 0, "blocks of one lane must share a swizzle");
  uint32_t voff0;
  uint32_t lds_wave;

  __device__ inline void init(int wave, int lane) {
    const int row0 = wave * ROWS_PER_BLK + lane / CH;
    const int p = lane % CH;
    const int c = p ^ (IS_V ? v8_swz<D>(row0) : k8_swz<D>(row0));
    voff0 = static_cast<uint32_t>(row0 * D + 16 * c);
    lds_wave = static_cast<uint32_t>(wave) * 1024u;
  }
  __device__ inline void copy(const uint8_t* __restrict__ head, int k0, int N,
                              uint32_t stage_byte) const {
    const int rows = N - k0 > 0 ? N - k0 : 0;
    const auto rsrc = buffer_rsrc(head + static_cast<size_t>(k0) * D,
                                  static_cast<uint32_t>(rows) * static_cast<uint32_t>(D));
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      lds_dma16(rsrc, voff0 + i * (ROW_STEP * D), stage_byte + lds_wave + i * 4096u);
  }
};

__device__ inline i32x2 lds_read_tr_b8(uint32_t byte) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(IOFA_LDS(i32x2, static_cast<uintptr_t>(byte)));
}

// One wave's share of the recurrence (32 query rows).
template <int D>
struct Fp8Wave {
  using C = Fp8Cfg<D>;
  i32x8 qf[C::KB];            // Q fragments (B operand of S^T = K Q^T)
  f32x16 o[C::CB];            // O^T accumulator: lane owns one query column
  float m_run;                // reference maximum, log2 units
  float l_run;                // this lane half's share of the sum of p8 (the keys
                              // it holds), relative to m_run; the two halves are
                              // added in the epilogue
  int hi;                     // lane half
  uint32_t k_addr[C::KB][2];  // LDS byte addresses of K fragment halves, stage 0
  uint32_t v_addr[C::CB];     // LDS byte address of the first V^T read, stage 0

  __device__ inline void init_lanes(int lane, uint32_t sm) {
    const int l32 = lane & 31;
    hi = lane >> 5;
    // K: lane (l32, hi) holds key row l32 (+32 for the second score block),
    // bytes 64*kb + 32*hi .. +31, i.e. chunks 4*kb + 2*hi + {0, 1}.  The
    // same k-slot order is used for Q, so the products pair matching bytes.
    const int ksw = k8_swz<D>(l32);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        k_addr[kb][j] = sm + static_cast<uint32_t>(l32 * D + 16 * ((4 * kb + 2 * hi + j) ^ ksw));
    // V: ds_read_b64_tr_b8 -- in each 16-lane group, lane t supplies row
    // t/2 of an 8-row block, bytes 8*(t%2) .. +7 of a 16-byte column range,
    // and receives byte column t of the block's 8 rows.  Read u (0..3) of
    // lane (g = lane/16, t) covers keys 16u + 8*(e/4) + 4*hi + e%4 for
    // e = t/2 -- the keys P holds in k-slots 8u + e -- and columns
    // 32*cb + 16*(g%2) .. +15.
    const int g = lane >> 4, t = lane & 15, e = t >> 1;
    const int key = 8 * (e >> 2) + 4 * hi + (e & 3);
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
      const int chunk = 2 * cb + (g & 1);
      v_addr[cb] = sm + 2 * C::TB +
                   static_cast<uint32_t>(key * D + 16 * (chunk ^ v8_swz<D>(key)) + 8 * (t & 1));
    }
  }

  // Scores S^T of one tile (raw code dot products) from K stage S.
  template <int S>
  __device__ inline void scores(f32x16 (&s)[2]) const {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const uint32_t off = S * C::TB + sb * 32 * D;
        const u32x4 lo = lds_read16(k_addr[kb][0] + off);
        const u32x4 up = lds_read16(k_addr[kb][1] + off);
        const auto a = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        s[sb] = mfma_f8(a, qf[kb], s[sb]);
      }
    }
  }

  // acc += P V for one tile from V stage S.
  template <int S>
  __device__ inline void pv(const i32x8& pk) {
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
      const uint32_t a0 = v_addr[cb] + S * C::TB;
      const i32x2 r0 = lds_read_tr_b8(a0);
      const i32x2 r1 = lds_read_tr_b8(a0 + 16 * D);
      const i32x2 r2 = lds_read_tr_b8(a0 + 32 * D);
      const i32x2 r3 = lds_read_tr_b8(a0 + 48 * D);
      const i32x8 a = __builtin_shufflevector(__builtin_shufflevector(r0, r1, 0, 1, 2, 3),
                                              __builtin_shufflevector(r2, r3, 0, 1, 2, 3),
                                              0, 1, 2, 3, 4, 5, 6, 7);
      o[cb] = mfma_f8(a, pk, o[cb]);
    }
  }

  // Packs the 32 weights of a lane into E4M3: k-slot 16*sb + r (byte of the
  // operand) holds score block sb, register r.
  __device__ static inline void pack(const f32x16 (&p)[2], i32x8& pk) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x16& v = p[w >> 2];
      const int r0 = 4 * (w & 3);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[r0], v[r0 + 1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(v[r0 + 2], v[r0 + 3], word, true);
      pk[w] = word;
    }
  }

  // Tile maximum, reference update (moved whenever the tile's maximum is
  // above it), weights, row sum and packing.  Returns the rescale factor of
  // the older terms.  TAIL masks keys at or beyond keys_valid.
  template <bool TAIL>
  __device__ inline float softmax(f32x16 (&s)[2], i32x8& pk, float c2, int keys_valid) {
    float mraw = -__builtin_inff();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
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
    const float mt = mraw * c2;
    const bool move = mt > m_run;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
    m_run = move ? mt : m_run;
    const float msub = m_run - kP8Shift;
    float rs = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
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
    pack(s, pk);
    l_run = alpha * l_run + rs;
    return alpha;
  }

  // Weights against the current reference, packed; returns this lane's
  // partial sum (s is left intact for a redo).
  __device__ inline float softmax_lazy(const f32x16 (&s)[2], i32x8& pk, float c2) const {
    const float msub = m_run - kP8Shift;
    float rs = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x16& v = s[w >> 2];
      const int r0 = 4 * (w & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(v[r0], c2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(v[r0 + 1], c2, -msub));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(v[r0 + 2], c2, -msub));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(v[r0 + 3], c2, -msub));
      // the sum starts from its first term at d = 128 (saves an add of 0;
      // measured 0.9% faster there and no faster at d = 64)
      rs = (D == 128 && w == 0) ? p0 : rs + p0;
      rs += p1;
      rs += p2;
      rs += p3;
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pk[w] = word;
    }
    return rs;
  }
  // Accept the lazy tile (returns false) when every lane's partial sum (hence
  // every weight) is at most kP8Bound, else redo it against its own maximum
  // (returns true, with the rescale factor of the older terms in alpha).
  __device__ inline bool commit_lazy(float rs, f32x16 (&s)[2], i32x8& pk, float c2,
                                     float& alpha) {
    if (__all(rs <= kP8Bound)) {
      l_run += rs;
      return false;
    }
    alpha = softmax<false>(s, pk, c2, C::BC);
    return true;
  }

  __device__ inline void rescale(float alpha) {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) o[cb] *= alpha;
    }
  }
};

// Iteration j (parity P = j % 2) of the key sweep, as in the 16-bit kernel:
// copies of K_{j+2} into K stage P and V_j into V stage P at the top; the
// softmax of tile j interleaved with P_{j-1} V_{j-1} (V stage 1-P) and the
// scores of tile j+1 (K stage 1-P); a rescale of O if the reference moved,
// a wait for this iteration's copies and one barrier at the bottom.
template <int D>
__global__ __launch_bounds__(256, 2) void fa_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
    const uint8_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ Lse, int N,
    int num_qtiles, int num_wg, float c2, float v_scale, uint32_t qflip) {
  using C = Fp8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * C::TB];
  const uint32_t sm = lds_address(smem);
  const uint32_t kst[2] = {sm, sm + C::TB};
  const uint32_t vst[2] = {sm + 2 * C::TB, sm + 3 * C::TB};

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const GridPos gp = grid_pos(num_qtiles, 1, num_wg);
  const int bh = gp.bh, qt = gp.qt;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const uint8_t* Kh = K + head;
  const uint8_t* Vh = V + head;
  const int NT = (N + C::BC - 1) / C::BC;
  const bool ragged = (N % C::BC) != 0;

  Fp8TileCopy<D, false> kcp;
  Fp8TileCopy<D, true> vcp;
  kcp.init(wave, lane);
  vcp.init(wave, lane);
  kcp.copy(Kh, 0, N, kst[0]);
  kcp.copy(Kh, C::BC, N, kst[1]);

  Fp8Wave<D> ws;
  ws.init_lanes(lane, sm);
  const int q = qt * C::BR + wave * 32 + (lane & 31);
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    u32x4 lo = u32x4{0u, 0u, 0u, 0u}, up = lo;
    if (q < N) {
      const uint8_t* src = Q + head + static_cast<size_t>(q) * D + 64 * kb + 32 * ws.hi;
      lo = *reinterpret_cast<const u32x4*>(src);
      up = *reinterpret_cast<const u32x4*>(src + 16);
    }
    lo ^= qflip;
    up ^= qflip;
    ws.qf[kb] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) ws.o[cb] = f32x16{};
  ws.m_run = -__builtin_inff();
  ws.l_run = 0.f;

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa[2], sb[2];
  i32x8 pa, pb;
  ws.template scores<0>(sa);
  __syncthreads();   // K stage 0 is refilled in iteration 0

  constexpr int NM = C::CB + 2 * C::KB;         // products per iteration
  constexpr int NRD = 4 * C::KB + 4 * C::CB;    // LDS reads per iteration
  // vector instructions per product (d = 128: 10 measured 1.5-2% faster than
  // 14 with the raised issue priority; 6, 8, 12, 16 and 18 no faster)
  constexpr int VPM = D == 128 ? 10 : 28;
  // LDS reads issued ahead of the interleaved products (more is faster until
  // the registers they need run out)
  constexpr int LEAD = NRD < 16 ? NRD : 16;
  auto bottom = [&](float alpha) {
    ws.rescale(alpha);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto iteration = [&](auto par, int j, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], i32x8& p_prev,
                       i32x8& p_cur) {
    constexpr int P = decltype(par)::value;
    // raised issue priority from the copies through the products, dropped
    // before the wait and barrier (measured 1-4% faster, same output)
    __builtin_amdgcn_s_setprio(1);
    kcp.copy(Kh, (j + 2) * C::BC, N, kst[P]);
    vcp.copy(Vh, j * C::BC, N, vst[P]);
    const float rs = ws.softmax_lazy(s_cur, p_cur, c2);
    ws.template pv<1 - P>(p_prev);
    ws.template scores<1 - P>(s_nxt);
    // at d = 128 the reads stay 14 ahead for the whole tile (1.0% faster at
    // B2 H16 N4096, 1.8% at B1 H32 N16384 than 16 ahead draining over the
    // tile; 10 ahead 0.3% / 1.3%, 6 ahead slower)
    if constexpr (D == 128)
      interleave_mfma_valu_lead<NM, NRD, 14, VPM>();
    else
      interleave_mfma_valu<NM, NRD, LEAD, VPM>();
    // the redo decision is wave-uniform, so the accepted path (almost every
    // tile) carries no rescale factor and no rescale test
    float alpha;
    if (ws.commit_lazy(rs, s_cur, p_cur, c2, alpha)) ws.rescale(alpha);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto last = [&](auto par, int j, f32x16 (&s_cur)[2], i32x8& p_prev, i32x8& p_cur) {
    constexpr int P = decltype(par)::value;
    vcp.copy(Vh, j * C::BC, N, vst[P]);
    const float alpha = ragged ? ws.template softmax<true>(s_cur, p_cur, c2, N - j * C::BC)
                               : ws.template softmax<false>(s_cur, p_cur, c2, C::BC);
    if (j > 0) ws.template pv<1 - P>(p_prev);
    bottom(alpha);
    ws.template pv<P>(p_cur);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  if (NT == 1) {
    last(P0{}, 0, sa, pb, pa);
  } else {
    kcp.copy(Kh, 2 * C::BC, N, kst[0]);
    vcp.copy(Vh, 0, N, vst[0]);
    {
      const float alpha = ws.template softmax<false>(sa, pa, c2, C::BC);
      ws.template scores<1>(sb);
      interleave_mfma_valu<2 * C::KB, 4 * C::KB, 2, VPM>();
      bottom(alpha);
    }
    int j = 1;
    for (; j + 1 < NT - 1; j += 2) {
      iteration(P1{}, j, sb, sa, pa, pb);
      iteration(P0{}, j + 1, sa, sb, pb, pa);
    }
    if (j < NT - 1) {
      iteration(P1{}, j, sb, sa, pa, pb);
      last(P0{}, j + 1, sa, pb, pa);
    } else {
      last(P1{}, j, sb, pa, pb);
    }
  }

  // O = sv * acc / l in bf16; LSE = ln 2 * (m - 3 + log2 l).  Lane half hi
  // holds columns 32*cb + 8*g + 4*hi + 0..3 in registers 4*g .. 4*g+3.
  if (q < N) {
    const float l = halfwave_sum(ws.l_run);
    const float inv = v_scale / l;
    const float lse = (ws.m_run - kP8Shift + __builtin_amdgcn_logf(l)) * kLn2;
    uint16_t* Oq = O + head + static_cast<size_t>(q) * D;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = Bf16::pack(ws.o[cb][4 * g + 0] * inv, ws.o[cb][4 * g + 1] * inv);
        w[1] = Bf16::pack(ws.o[cb][4 * g + 2] * inv, ws.o[cb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(Oq + 32 * cb + 8 * g + 4 * ws.hi) = w;
      }
    }
    if (ws.hi == 0) Lse[static_cast<size_t>(bh) * N + q] = lse;
  }
}

template <int D>
hipError_t launch_fp8_d(const Fp8Args& a) {
  using C = Fp8Cfg<D>;
  const int num_qtiles = static_cast<int>((a.N + C::BR - 1) / C::BR);
  const int num_wg = static_cast<int>(a.BH) * num_qtiles;
  hipLaunchKernelGGL(fa_fwd_fp8_kernel<D>, dim3(num_wg), dim3(256), 0, a.stream,
                     static_cast<const uint8_t*>(a.Q), static_cast<const uint8_t*>(a.K),
                     static_cast<const uint8_t*>(a.V), static_cast<uint16_t*>(a.O), a.LSE,
                     static_cast<int>(a.N), num_qtiles, num_wg, a.c2, a.v_scale,
                     a.negate_q ? 0x80808080u : 0u);
  return hipGetLastError();
}

}  // namespace

int64_t fp8_workgroups(int64_t BH, int64_t N) {
  return BH * ((N + Fp8Cfg<128>::BR - 1) / Fp8Cfg<128>::BR);
}

hipError_t launch_fp8(const Fp8Args& a) {
  return a.d == 128 ? launch_fp8_d<128>(a) : launch_fp8_d<64>(a);
}

}  // namespace iofa
