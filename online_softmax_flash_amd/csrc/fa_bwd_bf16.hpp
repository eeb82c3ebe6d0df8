// Backward kernels, bf16 storage: the throughput path of the gradients.
//
// The gradients of exact softmax attention with every score block recomputed
// from Q, K and the forward's lse (fanfani.net "FlashAttention", section "The
// backward pass, and where the memory saving comes from"; synthetic.wiki
// "FlashAttention: attention's bottleneck is the wire, not the maths",
// section "The backward pass buys memory with recompute"), in three launches:
//
//  1. bwd_prep_bf16_kernel: D_i = dO_i . O_i and l2_i = lse_i * log2(e) per
//     query row, into the caller's workspace (so that P = exp2(s*c - l2)
//     costs one fma and one exp per score).
//  2. bwd_dkdv_bf16_kernel: one workgroup per (key block, K/V head,
//     sequence): S, P, dP, dS of every visible query block, dV += P^T dO and
//     dK += dS^T Q (four products per pair of blocks).
//  3. bwd_dq_bf16_kernel: one workgroup per (query block, query head,
//     sequence): S, P, dP, dS again and dQ += dS K (three products).
//
// Seven products per pair of blocks instead of the five the method needs:
// the alternative, dQ summed over key blocks by fp32 atomic adds from kernel
// 2, was built and measured on MI355X and is slower here (the atomic traffic,
// one fp32 dQ tile per pair of blocks, runs at about 2.7 TB/s; at B=1, H=32,
// N=8192 that is 4.4 GB, 1.6 ms against 0.6 ms for kernel 3).
//
// Shapes: Nq queries and Nk keys per sequence, the causal mask aligned to the
// bottom right (query i sees key j iff j <= i + Nk - Nq; a row that sees no
// key has O = 0, lse = -inf and zero gradients), uniform [B, H, N, d]
// batches or variable-length sequences packed along the token axis ([H, T,
// d] with cu_seqlens), as the general forward (fa_fwd_kv_bf16.hpp). The
// square backward is the case Nq = Nk.
//
// How the data reaches the matrix cores on gfx950:
//  * The streamed tiles (Q and dO in kernel 2, K and V in kernel 3) go from
//    global memory straight into LDS (global_load_lds), double-buffered:
//    block i+1 is in flight while block i is computed.
//  * Each tile is stored once, row-major, with rows padded by 16 bytes, and is
//    read two ways: 16-byte row reads where it is contracted over d (Q K^T,
//    dO V^T) and transposing reads (ds_read_b64_tr_b16) where it is contracted
//    over its rows (dO^T P, Q^T dS, K^T dS^T). No transposed copy is made.
//  * The 32 rows of every score tile are taken in the order rho below. With it
//    (a) the 16 fp32 accumulator values a lane holds are, as they stand, the
//    two 8-element fragments of the next product, (b) the 4 rows that one
//    16-lane group gathers in a transposing read are 4 rows apart, so with
//    16-byte padding both kinds of read are bank-conflict free, and (c) every
//    fragment address is a fixed offset from one per-lane base.
#pragma once

#include "fa_bwd.hpp"
#include "fa_fwd_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

// Row order of a 32-row score tile: index bits (b4 b3 b2 b1 b0) -> row
// 16*b4 + 4*(b1 b0) + 2*b3 + b2.
__device__ __forceinline__ constexpr int rho(int i) {
  return (i & 16) | ((i & 3) << 2) | (((i >> 3) & 1) << 1) | ((i >> 2) & 1);
}
// Row (within the 32-row tile) of accumulator element r of a lane of half h,
// when the tile's rows were taken in rho order: rho(8*(r/4) + 4*h + r%4).
__device__ __forceinline__ constexpr int rho_row(int r, int h) {
  return 16 * (r >> 3) + 4 * (r & 3) + 2 * ((r >> 2) & 1) + h;
}

// Direct copy of 64 per-row fp32 values (rows r0 .. r0+63 of one head, taken
// in rho order within each 32) into 256 bytes of LDS: lane l writes bytes
// 4l .. 4l+3. Rows >= N read row N-1 (the caller masks them). Issued through
// inline assembly like dma16 (the compiler does not track it, so it inserts
// no wait for it before later LDS accesses or fences): callers wait (vmcnt)
// and synchronise before the destination is read.
__device__ __forceinline__ void dma_row_stats(uint8_t* lds, const float* g, int r0, int N, int lane) {
  // The lane's row is recomputed at every call (a few instructions in one
  // wave) rather than kept across the caller's loop, where a spilled copy
  // reloaded from scratch would wait for the copies already in flight.
  asm volatile("" : "+v"(lane));
  int r = r0 + 32 * (lane >> 5) + rho(lane & 31);
  r = r < N ? r : N - 1;
  const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(lds));
  const uint64_t gs = uniform_u64((uint64_t)g);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(m0v), "v"((uint32_t)r * 4u), "s"(gs)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Workgroup barrier that orders LDS accesses only: waits for this wave's own
// LDS operations (lgkmcnt), not for its global loads or direct-to-LDS copies
// in flight, which a plain __syncthreads() would also wait for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Transposing read of a 16-bit fragment: two ds_read_b64_tr_b16, ROWB2 bytes apart.
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* p, int rows_apart_bytes) {
  const s16x4 lo = lds_read_tr(p);
  const s16x4 hi = lds_read_tr(p + rows_apart_bytes);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The extent of sequence b: query rows qs .. qs+nq-1 and key rows ks ..
// ks+nk-1 of each head, and the row strides of the batch and head axes.
struct SeqExtent {
  int qs, nq, ks, nk;
  long long q_bs, q_hs, k_bs, k_hs;
  __device__ __forceinline__ long long qrow0(int b, int hq) const { return b * q_bs + hq * q_hs + qs; }
  __device__ __forceinline__ long long krow0(int b, int hkv) const { return b * k_bs + hkv * k_hs + ks; }
};
__device__ __forceinline__ SeqExtent seq_extent(const BwdKvArgs& a, int b) {
  SeqExtent e{0, a.Nq, 0, a.Nk, (long long)a.Hq * a.Nq, a.Nq, (long long)a.Hkv * a.Nk, a.Nk};
  if (a.cu_q != nullptr) {
    // Offsets clamped into [0, total], lengths to the grid's maximum: any
    // offsets keep every access in bounds.
    e.qs = min(max(a.cu_q[b], 0), a.Nq);
    e.nq = min(min(max(a.cu_q[b + 1], e.qs), a.Nq) - e.qs, a.max_nq);
    e.ks = min(max(a.cu_k[b], 0), a.Nk);
    e.nk = min(min(max(a.cu_k[b + 1], e.ks), a.Nk) - e.ks, a.max_nk);
    e.q_bs = 0;
    e.k_bs = 0;
  }
  return e;
}

// Work item of workgroup wg: (sequence b, head h, block kb) out of HB = H*B
// (sequence, head) pairs times nb blocks, block-major (all pairs' block 0
// first). Uniform batches use decode_block's order (each XCD a contiguous
// range of pairs). Variable-length batches of more than 256 sequences (the
// others take compact_item's grid) take pair wg % HB, so that with
// round-robin dispatch over the 8 XCDs every XCD receives heads of every
// sequence: a long sequence's work is spread over the chip instead of
// landing on the XCD its pairs would occupy (every block of a pair still
// runs on one XCD).
__device__ __forceinline__ void decode_item(int wg, int H, int B, int nb, bool reverse, bool varlen, int& b, int& h,
                                            int& kb) {
  if (!varlen) {
    decode_block(wg, H, B, nb, reverse, b, h, kb);
    return;
  }
  const int HB = H * B;
  const int level = wg / HB, wp = wg % HB;
  b = wp / H;
  h = wp % H;
  kb = reverse ? (nb - 1 - level) : level;
}

// D = dO . O and l2 = lse * log2(e) per query row; one row per D/8 threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_bf16_kernel(BwdKvArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < a.rows) {
    const bf16x8 of = global_frag<uint16_t>(static_cast<const uint16_t*>(a.o) + row * D + part * 8);
    const bf16x8 gf = global_frag<uint16_t>(static_cast<const uint16_t*>(a.dout) + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)of[e], (float)gf[e], acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < a.rows && part == 0) {
    a.dsum[row] = acc;
    a.l2[row] = a.lse[row] * kLog2eF;
  }
}

// dK and dV: one workgroup per (block of 32*NP keys, K/V head, sequence), with
// 2*NP waves in NP pairs; pair p owns keys k0 + 32p .. +31 and splits the
// work of each 32-query subtile between its two waves:
//   wave p      ("P wave"):  S = Q K^T, P = exp2(S*c - l2) (masked), P -> LDS,
//                            then dV^T += dO^T P;            K and dV^T resident;
//   wave p + NP ("dS wave"): dP = dO V^T, then (P from LDS) dS = P (dP - D),
//                            dK^T += Q^T dS;                 V and dK^T resident.
// Each wave does 16 of the pair's 32 products per subtile and holds half of
// the pair's registers, so two waves fit on each SIMD and the softmax work of
// one overlaps the products of the other. Per block of 64 queries: barrier 1
// (block landed, previous block done), the P waves write P, barrier 2 (P
// visible; LDS only, the next block's copies stay in flight), the products
// that need P. Q, dO, l2 and D stream through LDS in double-buffered blocks,
// over every query head of the K/V head's group. No atomics: deterministic.
// LDS of the dK/dV kernel: two stages of (Q, dO, l2, D) and the P exchange.
template <int D, int NP>
struct DkdvLds {
  static constexpr int RS = 2 * D + 16;  // padded LDS row bytes
  static constexpr int TILE = 64 * RS;
  static constexpr int STAGE = 2 * TILE + 2 * 64 * 4;
  static constexpr int PX = 2 * 64 * 16 * 4;  // P exchange bytes per pair: 2 subtiles x 64 lanes x 16 fp32
  static constexpr int BYTES = 2 * STAGE + NP * PX;
};

// Work item wg of the dK/dV kernel, in `smem` (DkdvLds bytes, 1024-aligned).
template <int D, int NP, bool CAUSAL>
__device__ __forceinline__ void bwd_dkdv_body(const BwdKvArgs& a, uint8_t* smem, int wg) {
  constexpr int NW = 2 * NP;
  constexpr int BKV = 32 * NP, BQ = 64;
  constexpr int RS = DkdvLds<D, NP>::RS;
  constexpr int NF = D / 16, NDT = D / 32;
  constexpr int TILE = DkdvLds<D, NP>::TILE;
  constexpr int STAGE = DkdvLds<D, NP>::STAGE;
  constexpr int PX = DkdvLds<D, NP>::PX;
  typedef float f32x4 __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < NP;
  const int pair = pwave ? wave : wave - NP;
  const int h = lane >> 5, li = lane & 31;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int G = a.Hq / a.Hkv;
  const int nkb_max = (a.max_nk + BKV - 1) / BKV;
  int b, hkv, kb;
  if (a.compact) {
    // Variable length: the sequences' key blocks only, key block 0 (the most
    // work) first; XCD x takes K/V heads x, x + 8, ... when they divide by 8.
    const bool by_xcd = a.Hkv % 8 == 0;
    int j, cnt;
    if (!compact_item(wg, a.cu_k, a.B, a.Nk, a.max_nk, 1, BKV, a.Hkv, by_xcd, lane, b, j, kb, cnt))
      return;  // grid padding; uniform over the workgroup
    hkv = by_xcd ? wg % 8 + 8 * j : j;
  } else {
    decode_item(wg, a.Hkv, a.B, nkb_max, false, a.cu_q != nullptr, b, hkv, kb);  // key block 0 has the most work
  }
  const SeqExtent sq = seq_extent(a, b);
  const int nq = sq.nq, nk = sq.nk;
  const int k0 = kb * BKV;
  if (k0 >= nk) return;  // uniform over the workgroup: no barrier reached yet
  const int off = CAUSAL ? nk - nq : 0;  // causal: query i sees key j iff j <= i + off
  const int kw0 = k0 + pair * 32;
  const int kj = kw0 + li;  // this lane's key
  const long long krow0 = sq.krow0(b, hkv);

  // Steps: (query head g of the group, query block), from the first query
  // block any key of this workgroup is visible to. A sequence without
  // queries has no steps: its dK and dV are 0.
  const int nqb = (nq + BQ - 1) / BQ;
  const int qb_start = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int nqs = nq > 0 ? max(nqb - qb_start, 0) : 0;
  const int nsteps = G * nqs;
  // The dS waves issue each step's copies (they wait for P at the second
  // barrier anyway); the P waves go straight on to their score products.
  // Copy offsets held per lane (BlockDma) with four pairs; recomputed per
  // call (LeanDma) with two (d = 256) or six, whose waves have no registers
  // to spare.
  constexpr bool HELD = NP == 4;
  const int cw = wave - NP;  // index among the dS waves; < 0 for the P waves
  BlockDma<D, BQ, RS, NP> dma;
  if constexpr (HELD) dma.init(cw >= 0 ? cw : 0, lane);
  auto copy_tile = [&](auto full_tag, uint8_t* dst, const uint16_t* src, int valid) {
    constexpr bool FULL = decltype(full_tag)::value;
    if constexpr (HELD)
      dma.template issue<FULL>(dst, src, valid, cw);
    else
      LeanDma<D, BQ, RS, NP>::template issue<FULL>(dst, src, valid, cw, lane);
  };
  auto prefetch = [&](int i) {
    if (pwave) return;
    const int g = i / nqs, q0 = (qb_start + i % nqs) * BQ;
    const long long qr = sq.qrow0(b, hkv * G + g);
    uint8_t* st = smem + (i & 1) * STAGE;
    const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + (qr + q0) * D;
    const uint16_t* Og = static_cast<const uint16_t*>(a.dout) + (qr + q0) * D;
    if (q0 + BQ <= nq) {
      copy_tile(std::true_type{}, st, Qg, BQ);
      copy_tile(std::true_type{}, st + TILE, Og, BQ);
    } else {
      copy_tile(std::false_type{}, st, Qg, nq - q0);
      copy_tile(std::false_type{}, st + TILE, Og, nq - q0);
    }
    if (cw == 0) dma_row_stats(st + 2 * TILE, a.l2 + qr, q0, nq, lane);
    if (cw == NP - 1) dma_row_stats(st + 2 * TILE + BQ * 4, a.dsum + qr, q0, nq, lane);
  };
  if (nsteps > 0) prefetch(0);

  // This wave's resident operand: K (P wave) or V (dS wave), 32 keys, as
  // B-operand fragments; and its accumulator, dV^T or dK^T.
  const uint16_t* KV = static_cast<const uint16_t*>(pwave ? a.k : a.v) + krow0 * D;
  bf16x8 kvf[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    kvf[f] = (kj < nk) ? global_frag<uint16_t>(KV + (size_t)kj * D + 16 * f + 8 * h) : zero_frag<bf16x8>();
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = zero16();
  const float c = a.c;
  // Per-lane byte offsets: row reads (A operand, row rho(li), bytes 32f + 16h)
  // and transposing reads (16-lane group g16 gathers rows 4e + h (+2) of a
  // 16-row chunk, columns 32t + 16*(g16&1) + 4*(i16&3) .. +3).
  const int row_off = rho(li) * RS + 16 * h;
  const int tr_off = (4 * (i16 >> 2) + h) * RS + 32 * (g16 & 1) + 8 * (i16 & 3);
  // P exchange of this pair: [subtile][r/4][lane] x 4 fp32 (16 consecutive bytes per lane).
  uint8_t* px = smem + 2 * STAGE + pair * PX + 16 * lane;

  for (int i = 0; i < nsteps; ++i) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // barrier 1: step i has landed; every wave is done with step i-1
    if (i + 1 < nsteps) prefetch(i + 1);
    const int q0 = (qb_start + i % nqs) * BQ;
    const uint8_t* st = smem + (i & 1) * STAGE;
    const float* l2s = reinterpret_cast<const float*>(st + 2 * TILE);
    const float* dss = l2s + BQ;
    // Subtile sub (queries q0 + 32 sub ..) is needed unless it is past nq or
    // (causal) every key of the pair follows every query of it.
    const bool need0 = !CAUSAL || q0 + 31 + off >= kw0;
    const bool need1 = q0 + 32 < nq && (!CAUSAL || q0 + 63 + off >= kw0);
    // Both roles run the same products on role-selected tiles, so that the
    // accumulators stay in one set of registers:
    //   x = rows . kvf:     S = Q K^T (P wave) or dP = dO V^T (dS wave);
    //   acc += tr . bfr:    dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave).
    const uint8_t* qsm = st;
    const uint8_t* osm = st + TILE;
    const uint8_t* rows = pwave ? qsm : osm;
    const uint8_t* trs = pwave ? osm : qsm;
    // The products of a subtile are issued even when it is not needed (its
    // rows are in LDS either way; the result is then not used), so that in
    // the P wave subtile 1's products and subtile 0's exponentials sit in
    // one basic block and the scheduler can interleave them.
    f32x16 x[2];
    auto products = [&](int sub) {
      x[sub] = zero16();
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(x[sub], *reinterpret_cast<const bf16x8*>(rows + sub * 32 * RS + row_off + 32 * f), kvf[f]);
    };
    products(0);
    bf16x8 bfr[2][2];
    if (!pwave) products(1);
    if (pwave) {
      products(1);
      // P = exp2(S*c - l2) with masks; P to LDS for the dS wave; bf16 fragments.
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (!(sub ? need1 : need0)) continue;
        const int qs0 = q0 + 32 * sub;
        float p[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(l2s + 32 * sub + 8 * r4 + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) p[4 * r4 + e] = __builtin_amdgcn_exp2f(fmaf(x[sub][4 * r4 + e], c, -l4[e]));
        }
        // Masks: query row >= nq, key >= nk, or (causal) key > query + off.
        // A query that sees no key (lse = -inf) is masked on every key.
        if ((CAUSAL && qs0 + off < kw0 + 31) || qs0 + 32 > nq || kw0 + 32 > nk) {
          const int kd = kj - off - qs0 - h, nd = nq - qs0 - h;
          const bool kout = kj >= nk;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int base = rho_row(r, 0);
            if ((CAUSAL && kd > base) || nd <= base || kout) p[r] = 0.f;
          }
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = {p[4 * r4], p[4 * r4 + 1], p[4 * r4 + 2], p[4 * r4 + 3]};
          *reinterpret_cast<f32x4*>(px + sub * 4096 + r4 * 1024) = v;
        }
        pack_frag(bfr[sub][0], p);
        pack_frag(bfr[sub][1], p + 8);
      }
    }
    lds_barrier();  // barrier 2: P visible to the dS waves (the next step's copies stay in flight)
    if (!pwave) {
      // dS = P (dP - D) in bf16 fragments.
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (!(sub ? need1 : need0)) continue;
        float ds[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 p4 = *reinterpret_cast<const f32x4*>(px + sub * 4096 + r4 * 1024);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dss + 32 * sub + 8 * r4 + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[4 * r4 + e] = p4[e] * (x[sub][4 * r4 + e] - d4[e]);
        }
        pack_frag(bfr[sub][0], ds);
        pack_frag(bfr[sub][1], ds + 8);
      }
    }
    // acc += tr . bfr (contraction over the 32 queries of each subtile).
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (!(sub ? need1 : need0)) continue;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int t = 0; t < NDT; ++t)
          mma(acc[t], tr_frag(trs + sub * 32 * RS + tr_off + 16 * c2 * RS + 64 * t, 2 * RS), bfr[sub][c2]);
    }
  }

  if (kj < nk) {
    // P waves hold dV^T, dS waves dK^T (times scale): rows = d, column = key li.
    uint16_t* out = static_cast<uint16_t*>(pwave ? a.dv : a.dk) + (krow0 + kj) * D;
    const float mul = pwave ? 1.f : a.scale;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint16_t ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(acc[t][4 * gq + e] * mul, ov[e]);
        *reinterpret_cast<uint2*>(out + 32 * t + 8 * gq + 4 * h) = *reinterpret_cast<const uint2*>(ov);
      }
  }
}

// dQ: one workgroup per (block of 32*NW queries, query head, sequence). Each
// wave keeps 32 query rows of Q and dO as B-operand fragments in registers and
// accumulates dQ^T over the visible key blocks; K and V stream through LDS in
// blocks of 64 keys.
// LDS of the dQ kernel: two stages of (K, V) blocks of 64 keys.
template <int D>
struct DqLds {
  static constexpr int RS = 2 * D + 16;
  static constexpr int TILE = 64 * RS;
  static constexpr int STAGE = 2 * TILE;
  static constexpr int BYTES = 2 * STAGE;
};

// Work item wg of the dQ kernel, in `smem` (DqLds bytes, 1024-aligned).
template <int D, int NW, bool CAUSAL>
__device__ __forceinline__ void bwd_dq_body(const BwdKvArgs& a, uint8_t* smem, int wg) {
  constexpr int BM = 32 * NW, BK = 64;
  constexpr int RS = DqLds<D>::RS;
  constexpr int NF = D / 16, NDT = D / 32;
  constexpr int TILE = DqLds<D>::TILE;
  constexpr int STAGE = DqLds<D>::STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  // Wave index in a scalar register: the per-wave tests below (causal skip,
  // masked subtile) are then branches, not per-lane predication.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int nqb_max = (a.max_nq + BM - 1) / BM;
  int b, hq, qb;
  if (a.compact) {
    // Variable length: the sequences' query blocks only, the last (causal:
    // the most work) first; with K/V heads a multiple of 8, XCD x takes the
    // query heads of K/V heads x, x + 8, ..., whose K and V it then reads.
    const int G = a.Hq / a.Hkv;
    const bool by_xcd = a.Hkv % 8 == 0;
    int j, level, cnt;
    if (!compact_item(wg, a.cu_q, a.B, a.Nq, a.max_nq, 1, BM, a.Hq, by_xcd, lane, b, j, level, cnt))
      return;  // grid padding; uniform over the workgroup
    hq = by_xcd ? (wg % 8 + 8 * (j / G)) * G + j % G : j;
    qb = CAUSAL ? cnt - 1 - level : level;
  } else {
    decode_item(wg, a.Hq, a.B, nqb_max, CAUSAL, a.cu_q != nullptr, b, hq, qb);
  }
  // Uniform by construction; said so, so that the sequence's extents are
  // scalar loads and the masked-subtile test below stays a branch.
  b = __builtin_amdgcn_readfirstlane(b);
  hq = __builtin_amdgcn_readfirstlane(hq);
  qb = __builtin_amdgcn_readfirstlane(qb);
  const SeqExtent sq = seq_extent(a, b);
  const int nq = sq.nq, nk = sq.nk;
  const int q0 = qb * BM;
  if (q0 >= nq) return;  // uniform over the workgroup: no barrier reached yet
  const int off = CAUSAL ? nk - nq : 0;
  const int hkv = hq / (a.Hq / a.Hkv);
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + li;

  const long long qr = sq.qrow0(b, hq);
  const long long kr = sq.krow0(b, hkv);
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + qr * D;
  const uint16_t* dO = static_cast<const uint16_t*>(a.dout) + qr * D;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + kr * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + kr * D;

  // Key blocks up to the last key the workgroup's last query sees (none when
  // that query sees no key: dQ = 0).
  const int nkb = (nk + BK - 1) / BK;
  const int kmax = CAUSAL ? min(q0 + BM, nq) - 1 + off : nk - 1;
  const int kb_end = kmax < 0 ? 0 : min(nkb, kmax / BK + 1);
  BlockDma<D, BK, RS, NW> dma;
  dma.init(wave, lane);
  auto prefetch = [&](int kb) {
    uint8_t* st = smem + (kb & 1) * STAGE;
    const uint16_t* kg = K + (size_t)kb * BK * D;
    const uint16_t* vg = V + (size_t)kb * BK * D;
    if ((kb + 1) * BK <= nk) {
      dma.template issue<true>(st, kg, BK, wave);
      dma.template issue<true>(st + TILE, vg, BK, wave);
    } else {
      dma.template issue<false>(st, kg, nk - kb * BK, wave);
      dma.template issue<false>(st + TILE, vg, nk - kb * BK, wave);
    }
  };
  if (kb_end > 0) prefetch(0);

  bf16x8 qf[NF], of[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    qf[f] = (qi < nq) ? global_frag<uint16_t>(Q + (size_t)qi * D + 16 * f + 8 * h) : zero_frag<bf16x8>();
    of[f] = (qi < nq) ? global_frag<uint16_t>(dO + (size_t)qi * D + 16 * f + 8 * h) : zero_frag<bf16x8>();
  }
  const float l2 = (qi < nq) ? a.l2[qr + qi] : INFINITY;
  const float Di = (qi < nq) ? a.dsum[qr + qi] : 0.f;
  f32x16 dq_acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) dq_acc[t] = zero16();
  const float c = a.c;
  const int row_off = rho(li) * RS + 16 * h;
  const int tr_off = (4 * (i16 >> 2) + h) * RS + 32 * (g16 & 1) + 8 * (i16 & 3);

  for (int kb = 0; kb < kb_end; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < kb_end) prefetch(kb + 1);
    const uint8_t* st = smem + (kb & 1) * STAGE;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ks0 = kb * BK + 32 * sub;
      if (ks0 >= nk) break;
      if (CAUSAL && ks0 > qw0 + 31 + off) continue;  // every key follows every query of this wave
      const uint8_t* ks = st + sub * 32 * RS;
      const uint8_t* vs = ks + TILE;
      // S^T = K Q^T and dP^T = V dO^T: rows = keys (rho order), column = query li.
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(s, *reinterpret_cast<const bf16x8*>(ks + row_off + 32 * f), qf[f]);
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(dp, *reinterpret_cast<const bf16x8*>(vs + row_off + 32 * f), of[f]);
      // Masks: key >= nk, or (causal) key > query + off; a query that sees no
      // key (l2 = -inf) is masked on every key.
      const bool masked = (CAUSAL && ks0 + 31 > qw0 + off) || ks0 + 32 > nk;
      float ds[16];
      // Up to d = 128, two copies of the loop, so that unmasked subtiles
      // (most of them) carry no mask arithmetic. At d = 256, where a wave
      // holds 256 registers, the one loop below measured faster (the copies
      // cost 6% at wide_4k).
      if (D > 128) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l2));
          if (masked) {
            const int key = ks0 + rho_row(r, h);
            if (key >= nk || (CAUSAL && key > qi + off)) pv = 0.f;
          }
          ds[r] = pv * (dp[r] - Di);
        }
      } else if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l2));
          const int key = ks0 + rho_row(r, h);
          if (key >= nk || (CAUSAL && key > qi + off)) pv = 0.f;
          ds[r] = pv * (dp[r] - Di);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l2)) * (dp[r] - Di);
      }
      bf16x8 dsf[2];
      pack_frag(dsf[0], ds);
      pack_frag(dsf[1], ds + 8);
      // dQ^T += K^T dS^T (contraction over the 32 keys).
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int t = 0; t < NDT; ++t)
          mma(dq_acc[t], tr_frag(ks + tr_off + 16 * c2 * RS + 64 * t, 2 * RS), dsf[c2]);
    }
  }

  if (qi < nq) {
    uint16_t* dQ = static_cast<uint16_t*>(a.dq) + (qr + qi) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint16_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(dq_acc[t][4 * gq + e] * a.scale, out[e]);
        *reinterpret_cast<uint2*>(dQ + 32 * t + 8 * gq + 4 * h) = *reinterpret_cast<const uint2*>(out);
      }
  }
}

template <int D, int NP, bool CAUSAL>
__global__ __launch_bounds__(128 * NP) void bwd_dkdv_bf16_kernel(BwdKvArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DkdvLds<D, NP>::BYTES];
  bwd_dkdv_body<D, NP, CAUSAL>(a, smem, (int)blockIdx.x);
}

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void bwd_dq_bf16_kernel(BwdKvArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DqLds<D>::BYTES];
  bwd_dq_body<D, NW, CAUSAL>(a, smem, (int)blockIdx.x);
}

// dK/dV and dQ in one launch: workgroups [0, n_dkdv) take dK/dV items (the
// heaviest first), the rest dQ items, so that dQ work fills the compute units
// that the dK/dV kernel's last, longest items leave idle. The two are
// independent (both read D and l2 only). n_dkdv is a multiple of 8, so the
// XCD of a workgroup is that of its item index in either part.
template <int D, int NP, int NWQ, bool CAUSAL>
__global__ __launch_bounds__(128 * NP) void bwd_fused_bf16_kernel(BwdKvArgs a, int n_dkdv) {
  static_assert(128 * NP == 64 * NWQ, "one workgroup size for both parts");
  constexpr int L1 = DkdvLds<D, NP>::BYTES, L2 = DqLds<D>::BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L1 > L2 ? L1 : L2];
  const int wg = (int)blockIdx.x;
  if (wg < n_dkdv) bwd_dkdv_body<D, NP, CAUSAL>(a, smem, wg);
  else bwd_dq_body<D, NWQ, CAUSAL>(a, smem, wg - n_dkdv);
}

// The dQ kernel's instances live in their own translation unit (built with
// MFMA accumulators in VGPRs, which keeps it within two waves per SIMD).
hipError_t launch_bwd_dq_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream);
hipError_t launch_bwd_fused_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream);

template <int D, int NPKV, bool CAUSAL>
void launch_dkdv_bf16(const BwdKvArgs& a, hipStream_t stream) {
  constexpr int BKV = 32 * NPKV;
  // Compact variable-length grid: sum_s ceil(nk_s / BKV) <= Tk / BKV + B.
  const long long items = a.compact ? ((long long)a.Nk + BKV - 1) / BKV + a.B
                                    : (long long)((a.max_nk + BKV - 1) / BKV) * a.B;
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, NPKV, CAUSAL>), dim3((unsigned)(items * a.Hkv)), dim3(128 * NPKV), 0,
                     stream, a);
}

// D and l2, then the dK/dV kernel unless it runs in the fused launch.
template <int D, bool CAUSAL>
hipError_t launch_bwd_prep_dkdv_bf16(const BwdKvArgs& a, bool fused, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_prep_bf16_kernel<D>), dim3((unsigned)((a.rows + RPB - 1) / RPB)), dim3(256), 0, stream, a);
  if (fused) return hipGetLastError();
  // Pairs per workgroup: 4 (two waves per SIMD) while a wave's registers allow
  // it; at d = 256 a wave needs more than half the register file, so 2. At
  // d = 128 with the causal mask, 6 pairs (three waves per SIMD, 192 keys per
  // workgroup; the compiler keeps the wave within 168 registers with 2
  // spilled) when that still gives every compute unit four workgroups or more
  // to run one after another: 2-4% faster at 8192 tokens, slower on grids of
  // one or two rounds, where the larger workgroups leave the last round short.
  if constexpr (D == 128 && CAUSAL) {
    const long long wgs6 = (long long)((a.max_nk + 191) / 192) * a.Hkv * a.B;
    if (a.cu_q == nullptr && wgs6 >= 4LL * device_cu_count()) {
      launch_dkdv_bf16<D, 6, CAUSAL>(a, stream);
      return hipGetLastError();
    }
  }
  launch_dkdv_bf16<D, (D <= 128 ? 4 : 2), CAUSAL>(a, stream);
  return hipGetLastError();
}

}  // namespace fa
