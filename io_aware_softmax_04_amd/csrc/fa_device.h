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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct Bf16 {
  using vec8 = bf16x8;
  // fp32 value of the bf16 pattern in the low 16 bits of b
  __device__ static inline float to_f32(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static inline uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  // two floats -> two bf16 (round to nearest even) in one dword, lo first
  __device__ static inline uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  }
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct F16 {
  using vec8 = f16x8;
  __device__ static inline float to_f32(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
  __device__ static inline uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ static inline uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
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

// ------------------------------------------------------------ tile loads

// ------------------------------------------- swizzled LDS tiles (fused path)
//
// K and V tiles of BC rows x D 16-bit elements are copied from global memory
// straight into LDS with buffer_load_dwordx4 ... lds: one instruction moves
// 64 lanes x 16 bytes and writes them to 1 KiB of consecutive LDS bytes, lane
// l at byte 16*l.  The tiles keep their row-major order; within a row the
// 16-byte chunks are XOR-permuted so that the reads below hit 64 distinct
// banks:
//   K (read 16 B per lane, 16 rows per 16-lane group):
//       chunk c of row r sits at c ^ (r & 15)         (D = 128)
//                                c ^ ((r >> 1) & 7)   (D = 64)
//   V (read with ds_read_b64_tr_b16, 4 rows x 32 B per 16-lane group):
//       chunk c of row r sits at c ^ ((r & 3) << 2)          (D = 128)
//                                c ^ (((r >> 1) & 1) << 2)   (D = 64)
template <int D>
__device__ inline int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ inline int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// A tile read both ways -- 16-byte row fragments (16 consecutive rows, one
// chunk) and ds_read_b64_tr_b16 (aligned groups of 4 rows, two adjacent
// chunks) -- needs a swizzle whose 16 values over rows 0..15 are distinct
// (row reads) and whose values shifted right by one are distinct within
// every aligned group of 4 rows (transposed reads):
//       chunk c of row r sits at c ^ (((r & 3) << 2) | ((r >> 2) & 3))          (D = 128)
//                                c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))   (D = 64)
template <int D>
__device__ inline int kv_swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Swizzle selector of a tile copy: which of the layouts above.
enum SwzKind { kSwzK = 0, kSwzV = 1, kSwzKV = 2 };
template <int D>
__device__ inline int tile_swz(int kind, int row) {
  return kind == kSwzK ? k_swz<D>(row) : kind == kSwzV ? v_swz<D>(row) : kv_swz<D>(row);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define IOFA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// One buffer_load_dwordx4 ... lds: 64 lanes x 16 bytes, lane l from byte
// voff of the buffer `rsrc`, into 1 KiB of consecutive LDS bytes at
// lds_byte (lane l at lds_byte + 16*l).  Loads at or beyond the buffer's
// byte length return zeros.  Issued as inline assembly so the compiler does
// not track it: it would otherwise wait for every such copy before any LDS
// read (it cannot tell which LDS bytes a copy writes).  The caller orders it
// with explicit waits on the vector-memory counter before the copied bytes
// are read or the workgroup ends.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_byte)
               : "memory");
}
// The same copy marked non-temporal, for data that no other workgroup reads
// again (the caches then keep it for the shortest time).
__device__ inline void lds_dma16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_byte)
               : "memory");
}
// The same with 4 bytes per lane: 256 consecutive LDS bytes.
__device__ inline void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_byte)
               : "memory");
}

// Raw buffer over `bytes` bytes at p (range-checked loads; word 3 selects
// the 32-bit data format gfx9 buffers need for raw accesses).
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes),
                                           0x00020000);
}

__device__ inline uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(IOFA_LDS(const void, p)));
}

// Per-lane part of the direct copies of one K or V tile (BC rows x D 16-bit
// elements, row-major, chunks swizzled by the SwzKind SWZ) from global
// memory into an LDS stage by the NWV waves of a workgroup.  Wave w writes the 1 KiB blocks
// b = w + NWV*i (i = 0 .. PER_WAVE-1); with this interleave the swizzle of
// every row a lane copies is the same, and lane offsets differ between
// blocks only by a constant.  NT marks the copies non-temporal.
template <int D, int BC, int SWZ, int NWV = 4, bool NT = false>
struct TileCopy {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWS_PER_BLK = 64 / CH;     // rows in one 1 KiB block
  static constexpr int BLKS = BC * D * 2 / 1024;   // 1 KiB blocks per tile
  static constexpr int PER_WAVE = BLKS / NWV;
  static constexpr int ROW_STEP = NWV * ROWS_PER_BLK;  // rows between a lane's blocks
  static_assert(PER_WAVE * NWV == BLKS, "tile must split over the waves");
  static_assert(ROW_STEP % 16 == 0, "blocks of one lane must share a swizzle");
  uint32_t voff0;     // byte offset of this lane's chunk in block i = 0
  uint32_t lds_wave;  // byte offset of block i = 0 inside a stage (wave-uniform)

  // `wave` must be wave-uniform (read with readfirstlane by the caller).
  __device__ inline void init(int wave, int lane) {
    const int row0 = wave * ROWS_PER_BLK + lane / CH;
    const int p = lane % CH;
    const int c = p ^ tile_swz<D>(SWZ, row0);
    voff0 = static_cast<uint32_t>(row0 * D + 8 * c) * 2u;
    lds_wave = static_cast<uint32_t>(wave) * 1024u;
  }
  // Rows k0 .. k0+BC-1 of `head` (N rows) into the stage at LDS byte
  // address stage_byte.  Rows at or beyond N (also whole tiles past the
  // end) arrive as zeros.
  __device__ inline void copy(const uint16_t* __restrict__ head, int k0, int N,
                              uint32_t stage_byte) const {
    const int rows = N - k0 > 0 ? N - k0 : 0;
    const auto rsrc = buffer_rsrc(head + static_cast<size_t>(k0) * D,
                                  static_cast<uint32_t>(rows) * (D * 2u));
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      if constexpr (NT)
        lds_dma16_nt(rsrc, voff0 + i * (ROW_STEP * D * 2), stage_byte + lds_wave + i * (NWV * 1024u));
      else
        lds_dma16(rsrc, voff0 + i * (ROW_STEP * D * 2), stage_byte + lds_wave + i * (NWV * 1024u));
    }
  }
};

// 16-byte and transposing 8-byte LDS reads at a byte address.
__device__ inline u32x4 lds_read16(uint32_t byte) {
  return *IOFA_LDS(const u32x4, static_cast<uintptr_t>(byte));
}
__device__ inline s16x4 lds_read_tr8(uint32_t byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(IOFA_LDS(s16x4, static_cast<uintptr_t>(byte)));
}

template <class T>
__device__ inline typename T::vec8 lds_vec8(const uint16_t* p) {
  return __builtin_bit_cast(typename T::vec8, *reinterpret_cast<const u32x4*>(p));
}

template <class T>
__device__ inline typename T::vec8 gmem_vec8(const uint16_t* p) {
  return __builtin_bit_cast(typename T::vec8, *reinterpret_cast<const u32x4*>(p));
}

}  // namespace iofa
