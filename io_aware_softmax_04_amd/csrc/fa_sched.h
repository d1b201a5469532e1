// Scheduling and grid helpers shared by the fused forward kernels (16-bit
// and FP8 inputs).
#pragma once

#include "fa_device.h"

namespace iofa {

// Interleave, inside one scheduling region, NMFMA matrix products with the
// NDS LDS fragment reads they consume (LEAD reads first, the rest spread
// evenly) and the vector work of a softmax (VPM instructions per product).
template <int NMFMA, int R, int VPM, int I>
__device__ inline void interleave_step() {
  if constexpr (I < NMFMA) {
    constexpr int nrd = (I + 1) * R / NMFMA - I * R / NMFMA;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    if constexpr (nrd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nrd, 0);   // DS reads
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);       // VALU
    interleave_step<NMFMA, R, VPM, I + 1>();
  }
}
template <int NMFMA, int NDS, int LEAD, int VPM>
__device__ inline void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);        // DS reads
  interleave_step<NMFMA, NDS - LEAD, VPM, 0>();
}

// The same with the reads kept LEAD ahead of their consumers for the whole
// region: the products consume the NDS reads about evenly (NDS / NMFMA
// each), and before product k the reads issued are
// min(NDS, LEAD + ceil(k NDS / NMFMA)).  With interleave_mfma_valu the lead
// drains to nothing by the region's last products when NDS > NMFMA.
template <int NMFMA, int NDS, int LEAD, int VPM, int I>
__device__ inline void interleave_lead_step() {
  if constexpr (I < NMFMA) {
    constexpr auto issued = [](int k) {
      const int c = (k * NDS + NMFMA - 1) / NMFMA + LEAD;
      return c < NDS ? c : NDS;
    };
    constexpr int nrd = issued(I + 1) - issued(I);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    if constexpr (nrd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nrd, 0);   // DS reads
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);       // VALU
    interleave_lead_step<NMFMA, NDS, LEAD, VPM, I + 1>();
  }
}
template <int NMFMA, int NDS, int LEAD, int VPM>
__device__ inline void interleave_mfma_valu_lead() {
  __builtin_amdgcn_sched_group_barrier(0x100, LEAD < NDS ? LEAD : NDS, 0);   // DS reads
  interleave_lead_step<NMFMA, NDS, LEAD, VPM, 0>();
}

// Position of a workgroup in the grid.  The logical order (contiguous per
// XCD, see xcd_logical_id) is ((bh * splits) + split) * qtiles + qt, so the
// query tiles of one head and key range run side by side on one XCD and
// share its L2 copy of those keys and values.
struct GridPos {
  int bh, split, qt;
};
__device__ inline GridPos grid_pos(int num_qtiles, int num_splits, int num_wg) {
  const int L = xcd_logical_id(blockIdx.x, num_wg);
  const int rest = L / num_qtiles;
  return GridPos{rest / num_splits, rest % num_splits, L % num_qtiles};
}

// Keys of split s out of G: the whole BC-key tiles [s*NT/G, (s+1)*NT/G) of
// the NT tiles covering N keys (non-empty when G <= NT).  Returns the first
// key and the key count.
__device__ inline int2 key_range(int N, int BC, int split, int num_splits) {
  const int nt = (N + BC - 1) / BC;
  const int t0 = static_cast<int>(static_cast<int64_t>(split) * nt / num_splits);
  const int t1 = static_cast<int>(static_cast<int64_t>(split + 1) * nt / num_splits);
  const int kbeg = t0 * BC;
  const int kend = t1 * BC < N ? t1 * BC : N;
  return make_int2(kbeg, kend - kbeg);
}

}  // namespace iofa
