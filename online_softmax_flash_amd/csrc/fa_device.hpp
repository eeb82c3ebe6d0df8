// Device-side building blocks of the attention kernels (gfx950 / CDNA4).
//
// Matrix-core convention used by every kernel here: the 32x32 MFMA
// (v_mfma_f32_32x32x16_bf16, or eight v_mfma_f32_32x32x2_f32 in the fp32
// check mode) with one "fragment" of 8 elements per lane for each operand.
//   A operand: lane l holds row (l & 31) of A, 8 values of the contraction
//              index; B operand: lane l holds column (l & 31) of B, 8 values
//              of the contraction index. Which 8 contraction indices a lane
//              half (l >> 5) holds is the same function for A and B, so any
//              assignment of the 16 contraction indices to (half, element)
//              pairs gives the same product as long as A and B agree; the
//              kernels exploit that freedom to avoid data movement.
//   C/D (16 fp32 per lane): element r of lane l is C[row][col] with
//              col = l & 31 and row = 8*(r/4) + 4*(l>>5) + (r%4).
// Only the C layout is a hardware fact the kernels depend on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Storage element types: uint16_t holds bf16 bit patterns; float is the fp32
// check mode.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  using frag = bf16x8;
  static constexpr int kBytes = 2;
};
template <> struct Elem<float> {
  using frag = f32x8;
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// fp32 -> storage element (bf16: round to nearest even, via v_cvt_pk_bf16_f32).
__device__ __forceinline__ void to_elem(float x, uint16_t& out) {
  out = __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ void to_elem(float x, float& out) { out = x; }

__device__ __forceinline__ float elem_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}
__device__ __forceinline__ float elem_to_f32(float x) { return x; }

// Build a fragment from 8 fp32 values.
__device__ __forceinline__ void pack_frag(bf16x8& f, const float* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (__bf16)x[e];
}
__device__ __forceinline__ void pack_frag(f32x8& f, const float* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = x[e];
}

template <typename F> __device__ __forceinline__ F zero_frag() {
  F f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = 0;
  return f;
}

// Row permutation within each group of 16 rows: swaps bits 2 and 3 of the row
// index. If the rows of a score tile are taken in this order, the 16 fp32
// results a lane holds for one column (rows 8*(r/4) + 4*half + r%4) become,
// for r = 0..7 and r = 8..15, eight consecutive indices each
// (16*(r/8) + 8*half + r%8): exactly a fragment of the next product.
__device__ __forceinline__ int sigma(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// Index (within a 32-row tile) held by accumulator element r of a lane of
// half h, when the tile's rows were taken in sigma order.
__device__ __forceinline__ constexpr int sigma_row(int r, int h) {
  return 16 * (r >> 3) + 8 * h + (r & 7);
}

// A ROWS x ROW_BYTES tile in LDS, stored in 16-byte chunks with an XOR
// swizzle. Any 16 lanes that read the same logical chunk of 16 consecutive
// rows (aligned to 16) touch 16 distinct 16-byte bank groups, i.e. all 64
// banks once: no conflicts.
template <int ROWS, int ROW_BYTES>
struct SwzTile {
  static constexpr int kChunks = ROW_BYTES / 16;  // chunks per row
  static constexpr int kM = kChunks < 16 ? kChunks : 16;
  static constexpr int kRowsPer256 = 16 / kM;
  static constexpr int kBytes = ROWS * ROW_BYTES;
  static_assert(ROW_BYTES % 16 == 0, "rows must be whole 16-byte chunks");
  static_assert((kM & (kM - 1)) == 0, "chunks per row must be a power of two");
  __device__ __forceinline__ static int chunk(int row, int ch) {
    return row * kChunks + (ch ^ (((row / kRowsPer256) ^ (row >> 4)) & (kM - 1)));
  }
  __device__ __forceinline__ static int byte(int row, int ch) { return chunk(row, ch) * 16; }
};

// Read one fragment (8 elements starting at logical element col0 of row) from
// a swizzled tile.
template <typename T, typename Tile>
__device__ __forceinline__ typename Elem<T>::frag lds_frag(const uint8_t* base, int row, int col0) {
  using F = typename Elem<T>::frag;
  constexpr int FC = 8 * sizeof(T) / 16;  // 16-byte chunks per fragment
  const int ch0 = col0 * (int)sizeof(T) / 16;
  if constexpr (FC == 1) {
    return *reinterpret_cast<const F*>(base + Tile::byte(row, ch0));
  } else {
    F f;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 lo = *reinterpret_cast<const f32x4*>(base + Tile::byte(row, ch0));
    f32x4 hi = *reinterpret_cast<const f32x4*>(base + Tile::byte(row, ch0 + 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = lo[e];
      f[4 + e] = hi[e];
    }
    return f;
  }
}

// Read one fragment (8 consecutive elements) from global memory.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag global_frag(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::frag*>(p);
}

// Copy rows [0, ROWS) of a row-major global matrix with COLS elements per row
// into a swizzled tile, as 16-byte chunks; rows >= valid are zero-filled.
template <typename T, int ROWS, int COLS, int NT, typename Tile>
__device__ __forceinline__ void stage_rows(uint8_t* lds, const T* g, int valid, int tid) {
  constexpr int CPR = COLS * (int)sizeof(T) / 16;
  constexpr int TOTAL = ROWS * CPR;
  static_assert(TOTAL % NT == 0, "tile must split evenly over the threads");
#pragma unroll
  for (int it = 0; it < TOTAL / NT; ++it) {
    const int id = tid + it * NT;
    const int row = id / CPR, ch = id % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (row < valid) val = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(g) + ((size_t)row * COLS * sizeof(T) + ch * 16));
    *reinterpret_cast<uint4*>(lds + Tile::byte(row, ch)) = val;
  }
}

// Copy rows [0, ROWS) of a row-major global matrix (COLS elements per row)
// into a swizzled tile holding its transpose (COLS rows of ROWS elements);
// rows >= valid become zeros.
template <typename T, int ROWS, int COLS, int NT, typename TileT>
__device__ __forceinline__ void stage_rows_transposed(uint8_t* lds, const T* g, int valid, int tid) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int CPR = COLS / EPC;
  constexpr int TOTAL = ROWS * CPR;
  static_assert(TOTAL % NT == 0, "tile must split evenly over the threads");
#pragma unroll
  for (int it = 0; it < TOTAL / NT; ++it) {
    const int id = tid + it * NT;
    const int row = id / CPR, ch = id % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (row < valid) val = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(g) + ((size_t)row * COLS * sizeof(T) + ch * 16));
    const T* e = reinterpret_cast<const T*>(&val);
    const int b = row * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      *reinterpret_cast<T*>(lds + TileT::byte(ch * EPC + i, b / 16) + (b % 16)) = e[i];
    }
  }
}

}  // namespace fa
