// Device-side building blocks shared by the fused and the naive gfx950
// kernels: element types, the 32x32x16 MFMA wrappers, tile loaders into LDS,
// wave-half exchanges and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iofa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- types

struct Bf16 {
  using vec8 = bf16x8;
  __device__ static inline uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct F16 {
  using vec8 = f16x8;
  __device__ static inline uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Pack two 16-bit patterns into one dword (lo in bits 0..15).
__device__ inline uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// 16-bit element e (0..7) of a 16-byte chunk held as four dwords.
__device__ inline uint32_t half_of(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// ----------------------------------------------------- cross-lane helpers

// Combine a value with the same value of the lane 32 apart.  v_permlane32_swap
// exchanges the upper half-wave of its first operand with the lower half-wave
// of its second; fed the same value twice, each lane receives its own value
// in one result and its partner's in the other.
__device__ inline float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// --------------------------------------------------------- launch order

// Hardware dispatches consecutive workgroup ids round-robin over the 8 XCDs
// (each with its own L2).  Map hardware id w to a logical id so that each XCD
// receives a contiguous run of logical ids: consecutive query tiles of one
// head then run on one XCD and share its L2 copy of that head's K and V.
__device__ inline int xcd_logical_id(int w, int G) {
  constexpr int X = 8;
  const int q = G / X, rem = G % X;
  const int x = w % X, s = w / X;
  return x * q + (x < rem ? x : rem) + s;
}

// Position of key j (0..63 inside a 64-key tile) in a transposed V row, such
// that the 8 keys a lane multiplies in one 32x32x16 product of P V sit in 16
// consecutive bytes.  The score accumulator gives lane-half h, register r of
// a 32-key block the key 8*(r/4) + 4*h + r%4; taking registers 8*t .. 8*t+7
// as the k-slots of key step t swaps bits 2 and 3 of the key index.
__device__ inline int vt_pos(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// ------------------------------------------------------------ tile loads

// K (or Q) tile of BC rows x D 16-bit elements into LDS rows of stride KS
// elements.  Rows at or beyond `rows_valid` are filled with zeros.  256
// threads; each owns KCH 16-byte chunks; consecutive threads read consecutive
// chunks of one row (coalesced).
template <int D, int BC, int KS>
struct RowTile {
  static constexpr int CH = D / 8;
  static constexpr int KCH = BC * CH / 256;
  static_assert(KCH * 256 == BC * CH, "tile must split into 256 threads");
  u32x4 r[KCH];

  __device__ inline void load(const uint16_t* __restrict__ base, int rows_valid,
                              int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, cc = c % CH;
      if (row < rows_valid)
        r[i] = *reinterpret_cast<const u32x4*>(base + row * D + cc * 8);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
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

// V tile of BC keys x D 16-bit elements, stored transposed in LDS as D rows
// of stride VS elements (one row per output column c, keys along the row).
// Each thread loads KPB consecutive keys of one 16-byte column chunk and
// writes, for each of its 8 columns, KPB keys as one KPB*2-byte store.
// With PERM the keys are placed at vt_pos(j) (fused path, P from registers);
// otherwise in natural order (naive path, P from memory).  Keys at or beyond
// `rows_valid` are zeros.
template <int D, int BC, int VS, bool PERM>
struct VtTile {
  static constexpr int CH = D / 8;
  static constexpr int KPB = BC * CH / 256;
  static constexpr int NKG = BC / KPB;
  static_assert(KPB == 2 || KPB == 4, "unsupported V tile shape");
  u32x4 r[KPB];

  __device__ inline void load(const uint16_t* __restrict__ base, int rows_valid,
                              int tid) {
    const int kg = tid % NKG, cc = tid / NKG;
#pragma unroll
    for (int i = 0; i < KPB; ++i) {
      const int key = kg * KPB + i;
      if (key < rows_valid)
        r[i] = *reinterpret_cast<const u32x4*>(base + key * D + cc * 8);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
    const int kg = tid % NKG, cc = tid / NKG;
    const int j0 = kg * KPB;
    const int pos = PERM ? vt_pos(j0) : j0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = lds + (cc * 8 + e) * VS + pos;
      if constexpr (KPB == 4) {
        u32x2 w;
        w[0] = half_of(r[0], e) | (half_of(r[1], e) << 16);
        w[1] = half_of(r[2], e) | (half_of(r[3], e) << 16);
        *reinterpret_cast<u32x2*>(dst) = w;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = half_of(r[0], e) | (half_of(r[1], e) << 16);
      }
    }
  }
};

template <class T>
__device__ inline typename T::vec8 lds_vec8(const uint16_t* p) {
  return __builtin_bit_cast(typename T::vec8, *reinterpret_cast<const u32x4*>(p));
}

template <class T>
__device__ inline typename T::vec8 gmem_vec8(const uint16_t* p) {
  return __builtin_bit_cast(typename T::vec8, *reinterpret_cast<const u32x4*>(p));
}

}  // namespace iofa
