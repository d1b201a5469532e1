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
//   * workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//     query rows for the whole key sweep;
//   * the wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (fp32 acc): the
//     accumulator then gives each lane one query column, so the row max and
//     row sum are in-lane over 32 scores plus one exchange with the lane 32
//     apart (v_permlane32_swap);
//   * O^T = V^T P^T uses the same registers as the B operand (P rounded to
//     the input type), so P never leaves the lane; the rescale by
//     e^{m_old - m_new} and the final 1/l are in-lane too;
//   * K tiles (64 keys) sit row-major in LDS; V tiles sit transposed (one LDS
//     row per output column) so each lane reads its 8 keys as 16 bytes;
//   * K/V tiles are double-buffered: the next tile's global loads are in
//     flight while the current tile is multiplied; one barrier per tile;
//   * exponentials are exp2 with log2(e) folded into the fp32 scale.
#include "fa_device.h"
#include "fa_launch.h"

namespace iofa {

template <int D>
struct FusedCfg {
  static constexpr int NW = 4;            // waves per workgroup
  static constexpr int BR = 32 * NW;      // query rows per workgroup
  static constexpr int BC = 64;           // keys per tile
  static constexpr int KS = D + 8;        // K row stride in LDS (elements)
  static constexpr int VS = BC + 8;       // transposed-V row stride (elements)
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
};

template <class T, int D>
__global__ __launch_bounds__(256, 2) void fa_fwd_16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int N, int num_qtiles, int num_wg, float scale) {
  using C = FusedCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;

  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int bh = L / num_qtiles, qt = L % num_qtiles;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // a1: this lane's query row and its Q fragments (B operand of S^T = K Q^T)
  const int q = qt * C::BR + wave * 32 + l32;
  typename T::vec8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (q < N)
      qf[kk] = gmem_vec8<T>(Qh + static_cast<size_t>(q) * D + 16 * kk + 8 * hi);
    else
      qf[kk] = __builtin_bit_cast(typename T::vec8, u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) o[cb] = f32x16{};
  float m_run = -__builtin_inff();   // running max, log2 units of scaled scores
  float l_run = 0.f;                 // running denominator
  const float c2 = scale * kLog2e;

  RowTile<D, C::BC, C::KS> kt;
  VtTile<D, C::BC, C::VS, true> vt;
  const int ntiles = (N + C::BC - 1) / C::BC;

  // a2: first K/V tile into stage 0
  kt.load(Kh, N, tid);
  vt.load(Vh, N, tid);
  kt.store(smem, tid);
  vt.store(smem + C::K_ELEMS, tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * C::BC;
    const bool more = j + 1 < ntiles;
    if (more) {  // a2: next tile's global loads in flight during this tile
      kt.load(Kh + static_cast<size_t>(k0 + C::BC) * D, N - (k0 + C::BC), tid);
      vt.load(Vh + static_cast<size_t>(k0 + C::BC) * D, N - (k0 + C::BC), tid);
    }
    const uint16_t* Ks = smem + (j & 1) * C::STAGE;
    const uint16_t* Vt = Ks + C::K_ELEMS;

    // a3: S^T for 64 keys x 32 queries, two 32-key blocks
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const auto a = lds_vec8<T>(Ks + (32 * sb + l32) * C::KS + 16 * kk + 8 * hi);
        s[sb] = T::mfma(a, qf[kk], s[sb]);
      }
    }

    // scale into log2 units; keys beyond N get -inf (weight 0)
    float x[32];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[16 * sb + r] = s[sb][r] * c2;
    if (k0 + C::BC > N) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * sb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= N) x[16 * sb + r] = -__builtin_inff();
        }
    }

    // a4: row max over this tile, merged with the running max
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, x[i]);
    mx = halfwave_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float msub = (m_new == -__builtin_inff()) ? 0.f : m_new;

    // a5: exponentials, rescale factor, denominator
    const float alpha = __builtin_amdgcn_exp2f(m_run - msub);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = __builtin_amdgcn_exp2f(x[i] - msub);
      rs += x[i];
    }
    rs = halfwave_sum(rs);
    l_run = alpha * l_run + rs;
    m_run = m_new;

    // P rounded to the input type, as the B operand of four 16-key steps
    typename T::vec8 pk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack2(T::bits(x[8 * ks + 2 * e]), T::bits(x[8 * ks + 2 * e + 1]));
      pk[ks] = __builtin_bit_cast(typename T::vec8, w);
    }

    // a6: acc = alpha * acc + P V
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) o[cb] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const auto a = lds_vec8<T>(Vt + (32 * cb + l32) * C::VS + 16 * ks + 8 * hi);
        o[cb] = T::mfma(a, pk[ks], o[cb]);
      }
    }

    if (more) {
      uint16_t* nxt = smem + ((j + 1) & 1) * C::STAGE;
      kt.store(nxt, tid);
      vt.store(nxt + C::K_ELEMS, tid);
    }
    __syncthreads();
  }

  // a7: O = acc / l rounded to the input type; LSE = m + ln l (natural log)
  if (q < N) {
    const float inv_l = 1.0f / l_run;
    uint16_t* Oq = O + head + static_cast<size_t>(q) * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack2(T::bits(o[cb][4 * g + 0] * inv_l), T::bits(o[cb][4 * g + 1] * inv_l));
        w[1] = pack2(T::bits(o[cb][4 * g + 2] * inv_l), T::bits(o[cb][4 * g + 3] * inv_l));
        *reinterpret_cast<u32x2*>(Oq + 32 * cb + 8 * g + 4 * hi) = w;
      }
    }
    if (hi == 0)
      LSE[static_cast<size_t>(bh) * N + q] = (m_run + __builtin_amdgcn_logf(l_run)) * kLn2;
  }
}

// ---------------------------------------------------------------- fp32 path
//
// fp32 inputs keep every product and sum in fp32 on the vector ALUs (on
// MI355X the fp32 matrix and vector peaks are equal).  Workgroup = 32 query
// rows x 8 threads per row; each thread owns D/8 columns of q and of the
// output accumulator; a score is the 8-lane sum of partial dot products.
// K and V tiles of 32 keys are staged in LDS.

template <int D>
__global__ __launch_bounds__(256) void fa_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K,
    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
    int N, int num_qtiles, int num_wg, float scale) {
  constexpr int QPB = 32, TPQ = 8, DPT = D / TPQ, BC = 32, LS = D + 4;
  __shared__ __attribute__((aligned(16))) float Ks[BC * LS];
  __shared__ __attribute__((aligned(16))) float Vs[BC * LS];

  const int tid = threadIdx.x;
  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int bh = L / num_qtiles, qt = L % num_qtiles;
  const size_t head = static_cast<size_t>(bh) * N * D;
  const int qi = tid / TPQ, part = tid % TPQ;
  const int q = qt * QPB + qi;
  const int c0 = part * DPT;

  float qv[DPT], ov[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    qv[e] = (q < N) ? Q[head + static_cast<size_t>(q) * D + c0 + e] : 0.f;
    ov[e] = 0.f;
  }
  float m_run = -__builtin_inff(), l_run = 0.f;

  for (int k0 = 0; k0 < N; k0 += BC) {
    for (int i = tid; i < BC * D / 4; i += 256) {
      const int row = i / (D / 4), c4 = i % (D / 4);
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (k0 + row < N) {
        kv = *reinterpret_cast<const float4*>(K + head + static_cast<size_t>(k0 + row) * D + 4 * c4);
        vv = *reinterpret_cast<const float4*>(V + head + static_cast<size_t>(k0 + row) * D + 4 * c4);
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
      sc[j] = (k0 + j < N) ? part_dot * scale : -__builtin_inff();
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

  if (q < N) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) O[head + static_cast<size_t>(q) * D + c0 + e] = ov[e] / l_run;
    if (part == 0) LSE[static_cast<size_t>(bh) * N + q] = m_run + logf(l_run);
  }
}

// ------------------------------------------------------------- launchers

template <class T, int D>
static hipError_t launch16(const FwdArgs& a) {
  using C = FusedCfg<D>;
  const int qtiles = static_cast<int>((a.N + C::BR - 1) / C::BR);
  const int64_t wg = a.BH * qtiles;
  hipLaunchKernelGGL((fa_fwd_16_kernel<T, D>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                     a.stream, static_cast<const uint16_t*>(a.Q), static_cast<const uint16_t*>(a.K),
                     static_cast<const uint16_t*>(a.V), static_cast<uint16_t*>(a.O), a.LSE,
                     static_cast<int>(a.N), qtiles, static_cast<int>(wg), a.scale);
  return hipGetLastError();
}

template <int D>
static hipError_t launch32(const FwdArgs& a) {
  const int qtiles = static_cast<int>((a.N + 31) / 32);
  const int64_t wg = a.BH * qtiles;
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D>), dim3(static_cast<unsigned>(wg)), dim3(256), 0,
                     a.stream, static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                     static_cast<const float*>(a.V), static_cast<float*>(a.O), a.LSE,
                     static_cast<int>(a.N), qtiles, static_cast<int>(wg), a.scale);
  return hipGetLastError();
}

int64_t fused_workgroups(int dtype, int64_t BH, int64_t N) {
  const int64_t br = (dtype == kDtypeF32) ? 32 : FusedCfg<128>::BR;
  return BH * ((N + br - 1) / br);
}

hipError_t launch_fused(const FwdArgs& a) {
  if (a.dtype == kDtypeBF16) return a.d == 128 ? launch16<Bf16, 128>(a) : launch16<Bf16, 64>(a);
  if (a.dtype == kDtypeF16) return a.d == 128 ? launch16<F16, 128>(a) : launch16<F16, 64>(a);
  return a.d == 128 ? launch32<128>(a) : launch32<64>(a);
}

}  // namespace iofa
