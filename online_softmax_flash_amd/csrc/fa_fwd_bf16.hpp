// Forward kernel, bf16 storage: the throughput path.
//
// Same method as fwd_kernel (fa_fwd.hpp): the online-softmax recurrence of
// fanfani.net "FlashAttention", section "A pinch of math: making the softmax
// work in pieces", over one block of queries and a stream of key/value blocks
// (section "Do not materialize the matrix"). What differs is how the data
// reaches the matrix cores on gfx950:
//
//  * K and V blocks go from global memory straight into LDS
//    (global_load_lds_dwordx4), double-buffered: block j+1 is in flight while
//    block j is computed; one barrier per block.
//  * Both are kept row-major in LDS with padded rows (K: +16 bytes, V: +64
//    bytes). K is read as the A operand of S^T = K Q^T with 16-byte reads;
//    V is read as the A operand of O^T = V^T P^T with the transposing read
//    ds_read_b64_tr_b16, which hands each lane one column of a 4 x 16 block.
//    The padding makes both access patterns bank-conflict free and every
//    fragment address a fixed offset from one per-lane base.
//  * 8 waves x 32 query rows per workgroup (4 for d = 256): each K/V block
//    staged in LDS serves 256 queries.
//  * Rescaling is lazy: the reference maximum m used in exp2(s*c - m) is only
//    raised when a block's maximum exceeds it by more than TAU (log2 units),
//    so exponentials are at most 2^TAU and the O rescale (and its VALU work)
//    is skipped for most blocks. The final o / l is unchanged in exact
//    arithmetic: numerator and denominator always share the same reference.
//    Only an item's first block (and masked blocks) take the block maximum;
//    other blocks take the weights against the current reference directly
//    and check their sum (the rare block whose maximum jumped is computed
//    again), so the second score tile's products overlap the first tile's
//    exponentials.
//  * Causal: a wave whose 32 queries all precede a block skips its compute
//    (it still takes part in the block's loads and barrier).
//  * Persistent workgroups (d <= 128): one per CU, each running several work
//    items (query block, head, batch). During an item's last block the next
//    item's first K/V block and query rows are already loaded, so an item's
//    start-up latency hides behind the previous item's work (this matters
//    most for short sequences, with few blocks per item).
#pragma once

#include <atomic>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_fwd.hpp"

namespace fa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// Calls f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// LDS byte address (as used by ds_* instructions) of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The 2*NT transposing reads (ds_read_b64_tr_b16) that give the NT V fragments
// of one 16-key chunk, for O^T tiles t = 0..NT-1 (64 bytes apart), each
// fragment being rows +0..3 and +4..7 (ROWB bytes apart) of the chunk. Issued
// through inline assembly: the compiler does not insert waits for them, so
// wait<N>() must be called (LDS operations complete in order: lgkmcnt(N)
// leaves at most the N most recent ones in flight) before frag() is used.
template <int NT>
struct TrReads {
  s16x4 r[NT][2];
  template <int OFF, int ROWB>
  __device__ __forceinline__ void issue(uint32_t addr) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r[t][0]) : "v"(addr), "i"(OFF + 64 * t) : "memory");
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r[t][1]) : "v"(addr), "i"(OFF + 64 * t + 4 * ROWB) : "memory");
    }
  }
  template <int N>
  __device__ __forceinline__ void wait() {
    constexpr int n = N > 15 ? 15 : N;  // with more in flight, waiting for 15 is stricter, still correct
    if constexpr (NT == 4) {
      asm volatile("s_waitcnt lgkmcnt(%8)"
                   : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[1][0]), "+v"(r[1][1]), "+v"(r[2][0]), "+v"(r[2][1]),
                     "+v"(r[3][0]), "+v"(r[3][1])
                   : "i"(n));
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[t][0]), "+v"(r[t][1]) : "i"(n));
    }
  }
  __device__ __forceinline__ bf16x8 frag(int t) const {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[t][0], r[t][1], 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

template <int D, int BN, int NW>
struct Bf16FwdCfg {
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int KROW = 2 * D + 16;  // padded row bytes of the K block
  static constexpr int VROW = 2 * D + 64;  // padded row bytes of the V block
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = BN * VROW;
};

// Wave-uniform 64-bit value in scalar registers (readfirstlane returns int:
// convert through uint32_t so that the low half is zero-extended).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32) |
         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
}

// One direct global->LDS copy of 16 bytes per lane: lane i reads global
// gbase + voff (bytes) and writes LDS lds_base + 16*i. lds_base and gbase are
// wave-uniform (scalar registers; lds_base goes through M0). The compiler
// does not see this write to LDS: callers wait for it (vmcnt) and synchronise
// before the destination is read.
__device__ __forceinline__ void dma16(uint32_t lds_base, uint32_t voff, uint64_t gbase) {
  const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_base);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0v), "v"(voff), "s"(gbase)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Direct global->LDS copy of rows [0, BN) of a row-major bf16 [*, D] matrix
// into an LDS block with ROWB-byte rows (2*D data bytes + padding). The block
// is a sequence of 16-byte slots; wave-instruction n fills slots
// [64n, 64n + 64), lane i slot 64n + i, and this wave issues instructions
// n = wave, wave + NW, ... (the wave index is made scalar here, so these
// tests are branches); a lane whose slot is padding copies a data chunk of
// its row again, so no instruction needs a per-lane mask.
template <int D, int BN, int ROWB, int NW>
struct BlockDma {
  static constexpr int SPR = ROWB / 16;   // slots per row
  static constexpr int CPR = 2 * D / 16;  // data slots per row
  static constexpr int NINSTR = (BN * SPR + 63) / 64;
  static constexpr int NPER = (NINSTR + NW - 1) / NW;  // instructions per wave (upper bound)
  static_assert(BN * SPR % 64 == 0, "every copy instruction covers 64 slots of the block");
  // Byte offset of this lane's chunk within the block. A lane whose slot is
  // row padding copies the row's last data chunk again (the padding is never
  // read), so every lane of an instruction is active.
  uint32_t off[NPER];
  int row[NPER];  // the chunk's row, for clamping the ragged tail

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int n = wave + j * NW;
      const int slot = n * 64 + lane;
      const int r = slot / SPR, c = min(slot % SPR, CPR - 1);
      off[j] = (uint32_t)(r * D + c * 8) * 2u;
      row[j] = r;
    }
  }
  // Rows >= valid read row valid - 1 (finite data; the kernel masks those keys).
  // Issued in scalar-base form (block base address and LDS destination in
  // scalar registers, a 32-bit per-lane byte offset).
  template <bool FULL>
  __device__ __forceinline__ void issue(uint8_t* lds, const uint16_t* g, int valid, int wave_in) const {
    const int wave = __builtin_amdgcn_readfirstlane(wave_in);  // uniform: scalar tests and LDS bases
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(lds));
    const uint64_t gs = uniform_u64((uint64_t)g);
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int n = wave + j * NW;
      if (j * NW + NW <= NINSTR || n < NINSTR) {  // wave-uniform
        uint32_t e = off[j];
        if (!FULL && row[j] >= valid) e -= (uint32_t)((row[j] - valid + 1) * D * 2);
        dma16(lb + (uint32_t)n * 1024u, e, gs);
      }
    }
  }
};

// Direct global->LDS copy of rows [0, BN) of a row-major bf16 [*, D] matrix
// into BN rows of ROWB bytes, in the slot order of BlockDma (wave-instruction
// n fills 16-byte slots 64n .. 64n+63; padding slots are skipped), but with
// each lane's source offset recomputed at every call instead of held in
// registers: a workgroup of one wave issues all the block's instructions, and
// keeping their offsets would cost two registers per instruction.
template <int D, int BN, int ROWB, int NW>
struct LeanDma {
  static constexpr int SPR = ROWB / 16;
  static constexpr int CPR = 2 * D / 16;
  static constexpr int NINSTR = (BN * SPR + 63) / 64;
  // Whether the last instruction runs past the block (its lanes beyond the
  // block's last slot must stay inactive).
  static constexpr bool TAIL = BN * SPR % 64 != 0;
  template <bool FULL>
  __device__ __forceinline__ static void issue(uint8_t* lds, const uint16_t* g, int valid, int wave_in, int lane) {
    asm volatile("" : "+v"(lane));  // recompute below on every call
    const int wave = __builtin_amdgcn_readfirstlane(wave_in);  // uniform: scalar tests and LDS bases
    const uint64_t gs = uniform_u64((uint64_t)g);
#pragma unroll
    for (int n0 = 0; n0 < NINSTR; n0 += NW) {
      const int n = n0 + wave;
      if (n0 + NW <= NINSTR || n < NINSTR) {  // wave-uniform
        const int slot = n * 64 + lane;
        const int r = slot / SPR;
        // A lane whose slot is row padding copies its row's last data chunk
        // again (the padding is never read): no per-lane mask.
        const int c = min(slot - r * SPR, CPR - 1);
        if (!TAIL || n < NINSTR - 1 || r < BN) {
          const int rr = (!FULL && r >= valid) ? valid - 1 : r;
          dma16(lds_addr(lds) + (uint32_t)n * 1024u, (uint32_t)(rr * D + c * 8) * 2u, gs);
        }
      }
    }
  }
};

template <int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void fwd_bf16_kernel(FwdArgs a) {
  // Persistent workgroups (several items each) up to d = 128; at d = 256 (one
  // wave per SIMD, most registers in use) one item per workgroup measured
  // faster, and the item loop compiles away.
  constexpr bool PERSIST = D <= 128;
  using C = Bf16FwdCfg<D, BN, NW>;
  constexpr int BM = C::BM;
  constexpr int NF = D / 16, NKT = BN / 32, NDT = D / 32, NKC = BN / 16;
  constexpr float TAU = 8.0f;
  constexpr float kTwoPowTau = 256.0f;  // 2^TAU
  constexpr int STAGE = C::KBYTES + C::VBYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int nqb = (N + BM - 1) / BM;
  const int nkb = (N + BN - 1) / BN;
  const int nfull_rows = N / BN;  // blocks with all BN rows inside [0, N)

  // Work items (query block, head, batch). The grid holds one workgroup per
  // CU; workgroup w takes items w, then in every other round the mirror
  // image of w among the workgroups of its XCD, so that long and short items
  // pair up (balanced causal work). Item i runs on XCD i mod 8. Persistent
  // workgroups of up to 8 waves take the (batch, head) pairs one at a time,
  // all of a pair's query blocks together (longest first), each XCD its own
  // eighth of the pairs when their count is a multiple of 8: the CUs of an
  // XCD then stream the same K and V through its L2 at the same time
  // (long_8k: 250 instead of 485 MB fetched per launch, time unchanged).
  // 16-wave workgroups (where the longer decode costs spills) and one-item
  // workgroups keep decode_block's order: level by level, longest first,
  // each XCD a contiguous range of pairs.
  const int G = (int)gridDim.x, n_items = nqb * a.Hq * a.B;
  auto item_of = [&](int r) {
    const int w = (int)blockIdx.x;
    const int ww = ((r & 1) && G % 8 == 0) ? (G / 8 - 1 - w / 8) * 8 + w % 8 : w;
    return r * G + ww;
  };
  struct Item {
    int b, hq, q0, kb_end, kb_full;
  };
  auto make_item = [&](int it) {
    Item x;
    int qb;
    if constexpr (PERSIST && NW <= 8) {  // (16-wave workgroups at 128 registers: decode_block)
      // XCD x takes pairs x * HB/8 .. (x+1) * HB/8 - 1 (HB a multiple of 8;
      // otherwise the items of a pair simply follow one another).
      const unsigned HB = (unsigned)(a.Hq * a.B), X = HB % 8u == 0 ? 8u : 1u;
      const unsigned xcd = (unsigned)it % X, j = (unsigned)it / X;
      const unsigned p = xcd * (HB / X) + j / (unsigned)nqb, level = j % (unsigned)nqb;
      x.b = (int)(p / (unsigned)a.Hq);
      x.hq = (int)(p % (unsigned)a.Hq);
      qb = CAUSAL ? nqb - 1 - (int)level : (int)level;
    } else {
      decode_block(it, a.Hq, a.B, nqb, CAUSAL, x.b, x.hq, qb);
    }
    x.q0 = qb * BM;
    const int q_last = min(x.q0 + BM, N) - 1;
    x.kb_end = CAUSAL ? min(nkb, q_last / BN + 1) : nkb;
    // Blocks [0, kb_full) need no mask for any query of the workgroup: every
    // key is < N and (causal) <= the first query q0.
    x.kb_full = CAUSAL ? min((x.q0 + 1) / BN, N / BN) : N / BN;
    return x;
  };

  // With 8 or 16 waves the block copies are issued by the last four only,
  // one per SIMD (the SIMD's other waves go on computing while these stall
  // on the issue): 2% faster at long_8k, 1-3% on shorter shapes, than every
  // wave issuing its share; the first four waves as the issuers gained less
  // (0.8%). With 16 waves (d = 64, 128 registers a wave) the four issuers
  // recompute their offsets per call (LeanDma), which also ends the
  // compiler's spills there: d = 64 causal 2.6-9% faster.
  constexpr int CW = NW >= 8 ? 4 : NW;
  const int cwave = wave - (NW - CW);  // index among the issuing waves; < 0 for the others
  constexpr bool LEAN = NW > 8;
  BlockDma<D, BN, C::KROW, CW> kdma;
  BlockDma<D, BN, C::VROW, CW> vdma;
  if constexpr (!LEAN) {
    kdma.init(cwave >= 0 ? cwave : 0, lane);
    vdma.init(cwave >= 0 ? cwave : 0, lane);
  }
  // Block kb of item x into LDS stage st (0 or 1).
  auto copy_block = [&](const Item& x, int kb, int st_idx) {
    uint8_t* st = smem + st_idx * STAGE;
    const size_t off = ((size_t)(x.b * a.Hkv + x.hq / (a.Hq / a.Hkv)) * N + (size_t)kb * BN) * D;
    const uint16_t* kg = static_cast<const uint16_t*>(a.k) + off;
    const uint16_t* vg = static_cast<const uint16_t*>(a.v) + off;
    if (cwave < 0) return;
    if constexpr (LEAN) {
      if (kb < nfull_rows) {
        LeanDma<D, BN, C::KROW, CW>::template issue<true>(st, kg, BN, cwave, lane);
        LeanDma<D, BN, C::VROW, CW>::template issue<true>(st + C::KBYTES, vg, BN, cwave, lane);
      } else {
        LeanDma<D, BN, C::KROW, CW>::template issue<false>(st, kg, N - kb * BN, cwave, lane);
        LeanDma<D, BN, C::VROW, CW>::template issue<false>(st + C::KBYTES, vg, N - kb * BN, cwave, lane);
      }
      return;
    }
    if (kb < nfull_rows) {
      kdma.template issue<true>(st, kg, BN, cwave);
      vdma.template issue<true>(st + C::KBYTES, vg, BN, cwave);
    } else {
      kdma.template issue<false>(st, kg, N - kb * BN, cwave);
      vdma.template issue<false>(st + C::KBYTES, vg, N - kb * BN, cwave);
    }
  };
  bf16x8 qf[NF];
  auto load_q = [&](const Item& x) {
    const int q = x.q0 + wave * 32 + li;
    const uint16_t* Q = static_cast<const uint16_t*>(a.q) + (size_t)(x.b * a.Hq + x.hq) * N * D;
#pragma unroll
    for (int f = 0; f < NF; ++f)
      qf[f] = (q < N) ? global_frag<uint16_t>(Q + (size_t)q * D + 16 * f + 8 * h) : zero_frag<bf16x8>();
  };

  int round = 0;
  Item cur = make_item(item_of(0));  // the grid never exceeds the item count
  int base = 0;                      // blocks of earlier items: block kb of this item uses stage (base + kb) & 1
  copy_block(cur, 0, 0);             // in flight while the query rows are read
  load_q(cur);

  f32x16 oacc[NDT];
  float m_run, l_bf, l_32;
  const float c = a.c;
  for (;;) {
  const int q0 = cur.q0;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + li;
  const int kb_end = cur.kb_end, kb_full = cur.kb_full;
  const int next_item = item_of(round + 1);
  const bool has_next = PERSIST && next_item < n_items;
  auto prefetch = [&](int kb) { copy_block(cur, kb, (base + kb) & 1); };

#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = zero16();
  m_run = -INFINITY;  // reference maximum of s*c (log2 units)
  l_bf = 0.f;         // this lane's share of sum of the bf16-rounded weights (normalises O)
  l_32 = 0.f;         // this lane's share of sum of the fp32 weights (gives lse)

  // Per-lane byte offsets of the fragment reads.
  // K (A operand of S^T): row 32*kt + sigma(li), bytes 32*f + 16*h.
  const int k_off = sigma(li) * C::KROW + 16 * h;
  // V (A operand of O^T, transposing read): 16-lane group g = lane/16, i = lane%16
  // reads row 16*kc + 8*h + i/4 (+4 for elements 4..7), column 32*t + 16*(g&1) + 4*(i&3).
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_off = C::KBYTES + (8 * h + (i16 >> 2)) * C::VROW + 2 * (16 * (g16 & 1) + 4 * (i16 & 3));

  // One key block: S^T = K Q^T, online-softmax update, O^T += V^T P^T.
  // after_scores() runs once the score products are issued (at once when the
  // wave skips the block): in the item's last block it reads the next item's
  // query rows, whose registers the products no longer need.
  auto block = [&](int kb, auto masked_tag, auto&& after_scores) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = kb * BN;
    if (CAUSAL && k0 > qw0 + 31) {  // every key of the block follows every query of this wave
      after_scores();
      return;
    }
    const uint8_t* st = smem + ((base + kb) & 1) * STAGE;
    f32x16 s[NKT];
    auto scores = [&] {
      bf16x8 kf[NKT][NF];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int f = 0; f < NF; ++f) kf[kt][f] = *reinterpret_cast<const bf16x8*>(st + k_off + 32 * kt * C::KROW + 32 * f);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        s[kt] = zero16();
#pragma unroll
        for (int f = 0; f < NF; ++f) mma(s[kt], kf[kt][f], qf[f]);
      }
      // Schedule: the first tile's K reads, then each later read paired with
      // one product, then the remaining products -- reads run ahead of use.
      {
        __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
#pragma unroll
        for (int i = 0; i < (NKT - 1) * NF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
      }
    };
    bool keep[NKT][16];
    auto mask = [&] {
      if constexpr (MASKED) {
        // Key k0 + 32 kt + sigma_row(r, h) is visible iff it is < N and
        // (causal) <= qi: one compare of a constant against the lane's limit.
        const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - k0 - 8 * h;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            keep[kt][r] = 32 * kt + sigma_row(r, 0) <= lim;
            if (!keep[kt][r]) s[kt][r] = -INFINITY;
          }
      }
    };
    // Raise the reference maximum if the block's maximum exceeds it by more
    // than TAU; returns the factor by which o and l must be rescaled (1: none).
    auto raise_max = [&] {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxc = (mx == -INFINITY) ? -INFINITY : mx * c;
      float alpha = 1.f;
      if (__any(mxc > m_run + TAU)) {
        const float m_new = fmaxf(m_run, mxc);
        alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      return alpha;
    };
    // Weights exp2(s*c - m_run) in place; returns this lane's fp32 sum of them.
    auto weights = [&] {
      const float base = (m_run == -INFINITY) ? 0.f : m_run;
      float p32[2] = {0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -base));
          if constexpr (MASKED) p = keep[kt][r] ? p : 0.f;
          s[kt][r] = p;
          p32[r & 1] += p;
        }
      return p32[0] + p32[1];
    };
    // The item's first block sets the reference maximum. Later unmasked
    // blocks take the weights against the current reference first: every
    // weight is at most the lane's sum, so a sum <= 2^TAU shows that no score
    // exceeded the reference by more than TAU (the condition for raising it).
    // Otherwise (rare: the maximum jumped; an overflowed weight gives an
    // infinite sum) the block's scores are computed again and the reference
    // raised first, which is the decision the block maximum would have taken:
    // the results are those of taking the maximum in every block.
    float psum, alpha = 1.f;
    bool slow = (kb == 0) || MASKED;
    if (!slow) {
      // Unmasked later block: the products of the second score tile run
      // while the weights of the first are taken.
      scores();
      psum = weights();
      {
        // K reads, then tile 0's products, then tile 1's products each
        // followed by a share of tile 0's weight arithmetic.
        __builtin_amdgcn_sched_group_barrier(0x100, NF, 1);
        for (int i = 0; i < (NKT - 1) * NF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        }
        for (int i = 0; i < NF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
        }
      }
      slow = __any(!(psum <= kTwoPowTau));
    }
    if (slow) {
      asm volatile("" ::: "memory");  // read K again (the first reads are not kept live)
      scores();
      mask();
      alpha = raise_max();
      psum = weights();
    }
    after_scores();
    if (__any(alpha != 1.f)) {
      l_bf *= alpha;
      l_32 *= alpha;
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
    }
    l_32 += psum;
    // P rounded to bf16 (the B operand of P V). O is normalised by the sum of
    // these same rounded weights (v_dot2 against (1, 1)), so o / l is an exact
    // convex combination of the weights the matrix cores used.
    uint32_t pw[NKC][4];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {(__bf16)s[kc >> 1][8 * (kc & 1) + 2 * e], (__bf16)s[kc >> 1][8 * (kc & 1) + 2 * e + 1]};
        pw[kc][e] = __builtin_bit_cast(uint32_t, pr);
      }
    float pbf[2] = {0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pbf[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[kc][e]), kOnesBf16x2, pbf[e & 1], false);
    l_bf += pbf[0] + pbf[1];
    // O^T += V^T P^T. The V fragments of chunk kc+1 are requested before the
    // products of chunk kc; the reads are issued and waited for explicitly
    // (see TrReads), so the in-flight copy of the next block is never waited on.
    const uint32_t vaddr = lds_addr(st) + (uint32_t)v_off;
    constexpr bool VPIPE = true;  // double-buffer the V fragments (at d = 256 too: 390 of 512 registers)
    TrReads<NDT> vr[VPIPE ? 2 : 1];
    vr[0].template issue<0, C::VROW>(vaddr);
    static_for<0, NKC>([&](auto kcc) {
      constexpr int kc = decltype(kcc)::value;
      constexpr int cur = VPIPE ? (kc & 1) : 0;
      if constexpr (VPIPE && kc + 1 < NKC) {
        vr[(kc + 1) & 1].template issue<16 * (kc + 1) * C::VROW, C::VROW>(vaddr);
        vr[cur].template wait<2 * NDT>();
      } else {
        if constexpr (!VPIPE && kc > 0) vr[0].template issue<16 * kc * C::VROW, C::VROW>(vaddr);
        vr[cur].template wait<0>();
      }
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 w = {pw[kc][0], pw[kc][1], pw[kc][2], pw[kc][3]};
      const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
      for (int t = 0; t < NDT; ++t) mma(oacc[t], vr[cur].frag(t), pf);
    });
  };

  // After the barrier of block kb: the copy of block kb+1, or, in the last
  // block, of the next item's first block (into the stage just freed).
  auto after_barrier = [&](int kb) {
    if (kb + 1 < kb_end) prefetch(kb + 1);
    else if (has_next) copy_block(make_item(next_item), 0, (base + kb_end) & 1);
  };
  auto after_scores = [&](int kb) {
    if (kb + 1 == kb_end && has_next) load_q(make_item(next_item));
  };
  int kb = 0;
  for (; kb < kb_full; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // block kb has landed; every wave is done with block kb-1
    after_barrier(kb);
    block(kb, std::false_type{}, [&] { after_scores(kb); });
  }
  for (; kb < kb_end; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    after_barrier(kb);
    block(kb, std::true_type{}, [&] { after_scores(kb); });
  }

  // Epilogue: divide by the denominator once; lse in natural-log units.
  const float lb = l_bf + __shfl_xor(l_bf, 32);
  const float l32 = l_32 + __shfl_xor(l_32, 32);
  const float inv = 1.f / lb;
  if (qi < N) {
    uint16_t* O = static_cast<uint16_t*>(a.o) + (size_t)(cur.b * a.Hq + cur.hq) * N * D + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint16_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(oacc[t][4 * g + e] * inv, out[e]);
        *reinterpret_cast<uint2*>(O + 32 * t + 8 * g + 4 * h) = *reinterpret_cast<const uint2*>(out);
      }
    if (h == 0) a.lse[(size_t)(cur.b * a.Hq + cur.hq) * N + qi] = (m_run + __log2f(l32)) * 0.69314718055994531f;
  }
  if (!has_next) break;
  base += kb_end;
  cur = make_item(next_item);
  ++round;
  }
}

// Compute units of the current device, cached per device. The cache entries
// are atomics: concurrent first calls from several host threads each store
// the same value, so the library stays safe to call from any thread.
inline int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int BN, int NW, bool CAUSAL>
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  const long long items = (long long)((a.N + BM - 1) / BM) * a.Hq * a.B;
  const long long cap = D <= 128 ? device_cu_count() : items;  // one item per workgroup at d = 256
  const int grid = (int)(items < cap ? items : cap);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW, CAUSAL>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
