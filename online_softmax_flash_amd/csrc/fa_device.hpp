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
// swizzle of the chunk index by a function of the row. It is chosen so that
// (a) 16 lanes reading the same logical chunk of 16 consecutive rows (aligned
// to 16) touch 16 distinct 16-byte bank groups -- all 64 banks once -- and
// (b) for rows of 256 or 128 bytes, the 4 rows x 32 bytes that 16 lanes of a
// transposing read fetch (rows 4k..4k+3, logical chunks 2c and 2c+1) land in
// 8 distinct bank groups.
template <int ROWS, int ROW_BYTES>
struct SwzTile {
  static constexpr int kChunks = ROW_BYTES / 16;  // chunks per row
  static constexpr int kM = kChunks < 16 ? kChunks : 16;
  static constexpr int kRowsPer256 = 16 / kM;
  static constexpr int kBytes = ROWS * ROW_BYTES;
  static_assert(ROW_BYTES % 16 == 0, "rows must be whole 16-byte chunks");
  static_assert((kM & (kM - 1)) == 0, "chunks per row must be a power of two");
  // XOR applied to the chunk index of row `row` (an involution: applying it
  // to a physical chunk index gives back the logical one).
  __device__ __forceinline__ static int xr(int row) {
    if constexpr (kM == 16) {  // rows of >= 256 bytes: bits (b3 b2 b1 b0) -> (b3 b1 b0 b2)
      const int r = row & 15;
      return ((r & 8) | ((r & 3) << 1) | ((r >> 2) & 1)) ^ ((row >> 4) & 15);
    } else if constexpr (kM == 8) {  // 128-byte rows, two per 256 bytes: u = row/2, (u2 u1 u0) -> (u0 u2 u1)
      const int u = (row >> 1) & 7;
      return (((u & 1) << 2) | ((u >> 2) << 1) | ((u >> 1) & 1)) ^ ((row >> 4) & 7);
    } else {
      return ((row / kRowsPer256) ^ (row >> 4)) & (kM - 1);
    }
  }
  __device__ __forceinline__ static int chunk(int row, int ch) { return row * kChunks + (ch ^ xr(row)); }
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

// ---------------------------------------------------------------------------
// gfx950 LDS data movers (16-bit elements).

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Copy rows [0, ROWS) of a row-major bf16 matrix (COLS elements per row) into
// a swizzled LDS tile with direct global->LDS loads (global_load_lds_dwordx4):
// each lane of a wave writes 16 bytes at LDS base + 16*lane, so the lane's
// global address is chosen to be the chunk that the swizzled layout puts
// there. Rows >= valid read row valid-1 instead (finite values; the caller
// masks them). Completion is tracked by vmcnt; callers wait before reading.
template <int ROWS, int COLS, int NT>
__device__ __forceinline__ void dma_rows_bf16(uint8_t* lds, const uint16_t* g, int valid, int wave, int lane) {
  using Tile = SwzTile<ROWS, COLS * 2>;
  constexpr int CPR = COLS * 2 / 16;
  constexpr int TOTAL = ROWS * CPR;
  static_assert(TOTAL % NT == 0, "tile must split evenly over the threads");
#pragma unroll
  for (int it = 0; it < TOTAL / NT; ++it) {
    const int base = it * NT + wave * 64;  // first LDS chunk written by this wave-instruction
    const int pc = base + lane;
    const int row = pc / CPR;
    const int ch = (pc % CPR) ^ Tile::xr(row);
    const int grow = row < valid ? row : valid - 1;
    const uint16_t* src = g + (size_t)grow * COLS + ch * 8;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds + base * 16), 16, 0, 0);
  }
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives element (i % 4) of the 4 elements loaded by lanes
// 4e + i/4, e = 0..3: if lanes 4e..4e+3 address the 16 consecutive elements
// of row e of a 4 x 16 block, lane i gets column i of rows 0..3.
__device__ __forceinline__ s16x4 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
}

// Item `item` of a compact grid over a variable-length batch: sequence s
// (rows cu[s] .. cu[s+1], clamped into [0, total] and to max_len rows, as the
// kernels clamp them) has cnt_s = ceil(len_s * mult / blk) blocks; the items
// run over sequences, then over block levels, then over the heads of the list
// (so that a sequence's heaviest blocks of every head come first). Up to 64
// sequences go longest first (ties in batch order), more in batch order. With
// xcd_heads (H a multiple of 8 and one item per workgroup in dispatch order),
// the items of XCD x = item % 8 are those of heads x, x + 8, ... only; the
// returned head index j then counts those heads (head = x + 8 * j). Every lane
// of the wave finds the sequence (by the item counts of the sequences ahead
// of each lane's, or by a prefix sum over chunks of 64 sequences) and returns
// the same, wave-uniform, values. False: grid padding.
__device__ __forceinline__ bool compact_item(long long item, const int* cu, int B, int total, int max_len, int mult,
                                             int blk, int H, bool xcd_heads, int lane, int& seq, int& j, int& level,
                                             int& cnt_seq) {
  const int hper = xcd_heads ? H / 8 : H;
  long long k = xcd_heads ? item / 8 : item;
  int s_found = -1, loc = 0, cnt_found = 1;
  if (B <= 64) {
    // Longest first, so that the longest sequences' items, which set the
    // critical path, start first (16 sequences of log-uniform lengths in
    // 64..4096 listed in random order: forward +1.8%, backward +0.8%; a batch
    // already in that order pays for the ranking, 1.5%).
    int n = -1, cnt = 0;
    if (lane < B) {
      const int s0 = min(max(cu[lane], 0), total);
      n = min(min(max(cu[lane + 1], s0), total) - s0, max_len);
      cnt = (int)(((long long)n * mult + blk - 1) / blk);
    }
    int ahead = 0;  // blocks of the sequences ahead of this lane's
    for (int t = 0; t < B; ++t) {
      const int nt = __builtin_amdgcn_readlane(n, t);
      const int ct = __builtin_amdgcn_readlane(cnt, t);
      ahead += ((nt > n) | ((nt == n) & (t < lane))) ? ct : 0;
    }
    const long long excl = (long long)ahead * hper;
    const unsigned long long hit = __ballot(lane < B && k >= excl && k < excl + (long long)cnt * hper);
    if (hit != 0) {
      const int l = __ffsll((long long)hit) - 1;
      s_found = l;
      loc = (int)(k - __shfl(excl, l));
      cnt_found = __shfl(cnt, l);
    }
  }
  for (int c0 = 0; c0 < B && B > 64; c0 += 64) {
    const int sb = c0 + lane;
    int cnt = 0;
    if (sb < B) {
      const int s0 = min(max(cu[sb], 0), total);
      const int n = min(min(max(cu[sb + 1], s0), total) - s0, max_len);
      cnt = (int)(((long long)n * mult + blk - 1) / blk);
    }
    long long incl = (long long)cnt * hper;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const long long excl = incl - (long long)cnt * hper;
    const unsigned long long hit = __ballot(k >= excl && k < incl);
    if (hit != 0) {  // uniform: k is the same in every lane
      const int l = __ffsll((long long)hit) - 1;
      s_found = c0 + l;
      loc = (int)(k - __shfl(excl, l));
      cnt_found = __shfl(cnt, l);
      break;
    }
    k -= __shfl(incl, 63);
  }
  if (s_found < 0) return false;
  seq = __builtin_amdgcn_readfirstlane(s_found);
  loc = __builtin_amdgcn_readfirstlane(loc);
  cnt_seq = __builtin_amdgcn_readfirstlane(cnt_found);
  level = loc / hper;
  j = loc % hper;
  return true;
}

}  // namespace fa
