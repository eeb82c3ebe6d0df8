// General forward, bf16 storage: rectangular problems (Nq queries, Nk keys,
// causal mask aligned to the bottom right), variable-length batches packed
// along the token axis, and split keys with a combine step.
//
// Per query row the kernel runs the same online-softmax recurrence as the
// square forward (fanfani.net "FlashAttention", section "A pinch of math:
// making the softmax work in pieces"), over the keys of one split only. With
// one split it writes O and lse directly. With several, each split writes its
// partial result (o / l in fp32, lse = m + ln l) and fwd_combine_kernel merges
// them with the recurrence's own rescale step: each partial enters like one
// block whose maximum is its lse and whose exponential sum is 1. That is the
// step that serves decoding (few queries, a long key/value cache: the cache,
// not the score matrix, is what limits serving -- fanfani.net, the closing
// paragraph of section "The backward pass, and where the memory saving comes
// from", and section "What to carry forward"), where one (batch, K/V head)
// alone cannot fill the chip.
//
// Rows. The G query heads that share a K/V head are packed into the rows of
// one workgroup: packed row r of (batch b, K/V head hkv) is query position
// r / G of query head hkv*G + r % G. A decode step (Nq = 1) thus fills G rows
// of a tile instead of one, and every K/V block staged in LDS serves all of
// them. Data movement is that of the square bf16 forward (fa_fwd_bf16.hpp):
// K and V blocks of 64 keys (32 for one-wave decoding workgroups) direct to
// LDS, double-buffered, padded rows, V read with transposing reads; Q rows in
// registers as B operands.
//
// Conventions: query i of a sequence with nq queries and nk keys sees key j
// iff j <= i + nk - nq (causal) and j < nk; a row that sees no key gets O = 0
// and lse = -inf.
#pragma once

#include "fa_fwd_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

// Copies of a K or V block: with several waves each lane's source offsets are
// computed once (BlockDma, a few registers); a one-wave decoding workgroup
// issues every instruction of the block and recomputes them per call
// (LeanDma), which keeps its registers free.
template <int D, int BN, int ROWB, int NW, bool HELD = (NW > 1)>
struct KvDma {
  BlockDma<D, BN, ROWB, NW> d;
  __device__ __forceinline__ void init(int wave, int lane) { d.init(wave, lane); }
  template <bool FULL>
  __device__ __forceinline__ void issue(uint8_t* lds, const uint16_t* g, int valid, int wave, int) const {
    d.template issue<FULL>(lds, g, valid, wave);
  }
};
template <int D, int BN, int ROWB, int NW>
struct KvDma<D, BN, ROWB, NW, false> {
  __device__ __forceinline__ void init(int, int) {}
  template <bool FULL>
  __device__ __forceinline__ void issue(uint8_t* lds, const uint16_t* g, int valid, int wave, int lane) const {
    LeanDma<D, BN, ROWB, NW>::template issue<FULL>(lds, g, valid, wave, lane);
  }
};

template <int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void fwd_kv_bf16_kernel(KvArgs a) {
  using C = Bf16FwdCfg<D, BN, NW>;
  constexpr int BM = C::BM;
  constexpr int NF = D / 16, NKT = BN / 32, NDT = D / 32, NKC = BN / 16;
  constexpr float TAU = 8.0f;
  constexpr float kTwoPowTau = 256.0f;  // 2^TAU
  constexpr int STAGE = C::KBYTES + C::VBYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int G = a.Hq / a.Hkv;
  // Work order. Workgroups are dispatched in linear-id order over the x-major
  // grid, round-robin over the 8 XCDs; the splits of one item are adjacent.
  // Uniform batches go level by level, heaviest row block first (causal: the
  // last row block sees the most keys), so that the longest items start
  // first; with one split and pairs a multiple of 8, each XCD receives a
  // contiguous range of (batch, K/V head) pairs, whose K and V then stay in
  // its L2. A variable-length batch goes sequence by sequence (up to 64
  // sequences: the longest first), heaviest row blocks of every head first
  // within each, over the row blocks its
  // sequences actually have (compact grid): a grid of max_seqlen row blocks
  // for every sequence spent
  // most of its workgroups on row blocks past the shorter sequences, each
  // dispatched only to read the offsets and exit.
  const long long wg = (long long)blockIdx.y * gridDim.x + blockIdx.x;
  const int HB = a.Hkv * a.B;
  const int split = (int)(wg % a.num_splits);
  const long long item = wg / a.num_splits;
  int b, hkv, rb;
  if (a.compact) {
    // Sequence s has ceil(n_s * G / BM) row blocks; items run over sequences,
    // then row-block levels (heaviest first), then K/V heads (compact_item).
    // With one split and K/V
    // heads a multiple of 8, the items of XCD x (item % 8, the dispatch
    // order) are those of heads x, x + 8, ... of every sequence, so each
    // head's K and V are read through one L2 (varlen_mix 285 -> 278 us);
    // every XCD still gets an equal share.
    const bool by_xcd = a.num_splits == 1 && a.Hkv % 8 == 0;
    int j, level, cnt_s;
    if (!compact_item(item, a.cu_q, a.B, a.Nq, a.max_nq, G, BM, a.Hkv, by_xcd, lane, b, j, level, cnt_s))
      return;  // grid padding; uniform over the workgroup
    hkv = by_xcd ? (int)(item % 8) + 8 * j : j;
    rb = CAUSAL ? cnt_s - 1 - level : level;
  } else {
    const int nrb = (int)(((long long)a.max_nq * G + BM - 1) / BM);
    if (item >= (long long)nrb * HB) return;  // grid padding; uniform over the workgroup
    int level, pair;
    if (a.cu_q != nullptr) {
      pair = (int)(item / nrb);
      level = (int)(item % nrb);
    } else {
      level = (int)(item / HB);
      const int wp = (int)(item % HB);
      pair = (a.num_splits == 1 && HB % 8 == 0) ? (wp % 8) * (HB / 8) + wp / 8 : wp;
    }
    b = pair / a.Hkv;
    hkv = pair % a.Hkv;
    rb = CAUSAL ? nrb - 1 - level : level;
  }

  // Sequence b: query rows qs .. qs+nq-1, key rows ks .. ks+nk-1 of each head.
  int qs = 0, nq = a.Nq, ks = 0, nk = a.Nk;
  long long q_bs = (long long)a.Hq * a.Nq, q_hs = a.Nq, k_bs = (long long)a.Hkv * a.Nk, k_hs = a.Nk;
  if (a.cu_q != nullptr) {
    // Offsets are clamped into [0, total] and lengths to the grid's maximum,
    // so that any offsets keep every access in bounds.
    qs = min(max(a.cu_q[b], 0), a.Nq);
    nq = min(min(max(a.cu_q[b + 1], qs), a.Nq) - qs, a.max_nq);
    ks = min(max(a.cu_k[b], 0), a.Nk);
    nk = min(max(a.cu_k[b + 1], ks), a.Nk) - ks;
    q_bs = 0;
    k_bs = 0;
  }
  const int nrows = nq * G;
  const int r0 = rb * BM;
  if (r0 >= nrows) return;  // uniform over the workgroup: no barrier reached yet

  // This lane's packed row: query i of head hkv*G + g.
  const int r = r0 + wave * 32 + li;
  const bool row_ok = r < nrows;
  const int i = r / G, hq = hkv * G + r % G;
  const long long row = (long long)b * q_bs + (long long)hq * q_hs + qs + i;  // also the lse / output row index
  const int off = nk - nq;  // causal: key j visible iff j <= i + off

  // Keys of this split, cut at the last key any row of the workgroup sees.
  const int i_last = min(nrows - 1, r0 + BM - 1) / G;
  int kend = min(nk, (split + 1) * a.split_keys);
  if (CAUSAL) kend = min(kend, i_last + off + 1);
  const int kbeg = split * a.split_keys;
  const int kb0 = kbeg / BN;
  const int kb_end = kend > kbeg ? (kend + BN - 1) / BN : kb0;
  // Blocks below kb_full need no mask: every key < kend and (causal) visible
  // to the workgroup's first row.
  const int i_first = r0 / G;
  int kfull = kend;
  if (CAUSAL) kfull = min(kfull, i_first + off + 1);
  const int kb_full = max(kb0, kfull / BN);
  // This wave's last row: blocks past its limit are skipped (causal).
  const int wlast = min(nrows - 1, r0 + wave * 32 + 31);
  const int wave_kmax = CAUSAL ? (wlast / G + off) : (kend - 1);

  const uint16_t* K = static_cast<const uint16_t*>(a.k) + ((long long)b * k_bs + (long long)hkv * k_hs + ks) * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + ((long long)b * k_bs + (long long)hkv * k_hs + ks) * D;

  // Eight-wave workgroups: the last four waves (one per SIMD) issue the
  // copies while the other four compute on, as in the square forward
  // (chunk_2k_8k +2.6%). With four waves every wave issues its share (two
  // or one issuing waves ran 20-30% slower).
  constexpr int CW = NW == 8 ? 4 : NW;
  const int cw = wave - (NW - CW);  // index among the issuing waves; < 0 for the others
  KvDma<D, BN, C::KROW, CW> kdma;
  KvDma<D, BN, C::VROW, CW> vdma;
  kdma.init(cw >= 0 ? cw : 0, lane);
  vdma.init(cw >= 0 ? cw : 0, lane);
  auto prefetch = [&](int kb) {
    if (cw < 0) return;
    uint8_t* st = smem + (kb & 1) * STAGE;
    const uint16_t* kg = K + (size_t)kb * BN * D;
    const uint16_t* vg = V + (size_t)kb * BN * D;
    const int valid = kend - kb * BN;
    if (valid >= BN) {
      kdma.template issue<true>(st, kg, BN, cw, lane);
      vdma.template issue<true>(st + C::KBYTES, vg, BN, cw, lane);
    } else {
      kdma.template issue<false>(st, kg, valid, cw, lane);
      vdma.template issue<false>(st + C::KBYTES, vg, valid, cw, lane);
    }
  };
  if (kb0 < kb_end) prefetch(kb0);

  bf16x8 qf[NF];
  const uint16_t* Qr = static_cast<const uint16_t*>(a.q) + row * D;
#pragma unroll
  for (int f = 0; f < NF; ++f) qf[f] = row_ok ? global_frag<uint16_t>(Qr + 16 * f + 8 * h) : zero_frag<bf16x8>();

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = zero16();
  float m_run = -INFINITY;
  float l_bf = 0.f, l_32 = 0.f;
  const float c = a.c;
  const int k_off = sigma(li) * C::KROW + 16 * h;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_off = C::KBYTES + (8 * h + (i16 >> 2)) * C::VROW + 2 * (16 * (g16 & 1) + 4 * (i16 & 3));
  const int klim = CAUSAL ? min(kend - 1, i + off) : kend - 1;  // last key this row sees

  auto block = [&](int kb, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = kb * BN;
    if (CAUSAL && k0 > wave_kmax) return;
    const uint8_t* st = smem + (kb & 1) * STAGE;
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
    };
    bool keep[NKT][16];
    auto mask = [&] {
      if constexpr (MASKED) {
        const int lim = klim - k0 - 8 * h;  // key k0 + 32 kt + sigma_row(e, h) is visible iff <= klim
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            keep[kt][e] = 32 * kt + sigma_row(e, 0) <= lim;
            if (!keep[kt][e]) s[kt][e] = -INFINITY;
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
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
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
        for (int e = 0; e < 16; ++e) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[kt][e], c, -base));
          if constexpr (MASKED) p = keep[kt][e] ? p : 0.f;
          s[kt][e] = p;
          p32[e & 1] += p;
        }
      return p32[0] + p32[1];
    };
    // The first block of the key range sets the reference maximum; masked
    // blocks take the block maximum too. Other blocks (every key visible to
    // every row, and every row already holds a finite reference, since the
    // visible keys of a row are a prefix) take the weights against the
    // current reference first: a lane sum <= 2^TAU shows that no score
    // exceeded the reference by more than TAU. Otherwise (rare) the scores
    // are computed again and the reference raised first, the decision the
    // block maximum would have taken.
    float psum, alpha = 1.f;
    bool slow = (kb == kb0) || MASKED;
    if (!slow) {
      scores();
      psum = weights();
      {
        // K reads, then tile 0's products, then the later tiles' products
        // each followed by a share of the weight arithmetic.
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
      {
        __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
#pragma unroll
        for (int i = 0; i < (NKT - 1) * NF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
      }
      mask();
      alpha = raise_max();
      psum = weights();
    }
    if (__any(alpha != 1.f)) {
      l_bf *= alpha;
      l_32 *= alpha;
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[t][e] *= alpha;
    }
    l_32 += psum;
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
    // V fragments of chunk kc+1 are requested before the products of chunk kc
    // (at d = 256 too: the registers fit without spills).
    const uint32_t vaddr = lds_addr(st) + (uint32_t)v_off;
    constexpr bool VPIPE = true;
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

  int kb = kb0;
  for (; kb < min(kb_full, kb_end); ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < kb_end) prefetch(kb + 1);
    block(kb, std::false_type{});
  }
  for (; kb < kb_end; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < kb_end) prefetch(kb + 1);
    block(kb, std::true_type{});
  }

  if (!row_ok) return;
  const float lb = l_bf + __shfl_xor(l_bf, 32);
  const float l32 = l_32 + __shfl_xor(l_32, 32);
  const bool seen = lb > 0.f;  // false: no key of this split is visible to the row
  const float inv = seen ? 1.f / lb : 0.f;
  const float lse_row = seen ? (m_run + __log2f(l32)) * 0.69314718055994531f : -INFINITY;
  if (a.num_splits == 1) {
    uint16_t* O = static_cast<uint16_t*>(a.o) + row * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint16_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(oacc[t][4 * gq + e] * inv, out[e]);
        *reinterpret_cast<uint2*>(O + 32 * t + 8 * gq + 4 * h) = *reinterpret_cast<const uint2*>(out);
      }
    if (h == 0) a.lse[row] = lse_row;
  } else {
    float* O = a.part_o + ((long long)split * a.rows + row) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float4 out;
        out.x = oacc[t][4 * gq + 0] * inv;
        out.y = oacc[t][4 * gq + 1] * inv;
        out.z = oacc[t][4 * gq + 2] * inv;
        out.w = oacc[t][4 * gq + 3] * inv;
        *reinterpret_cast<float4*>(O + 32 * t + 8 * gq + 4 * h) = out;
      }
    if (h == 0) a.part_lse[(long long)split * a.rows + row] = lse_row;
  }
}

// Merge of the split partials of every row: M = max_s lse_s, w_s = exp(lse_s - M),
// O = sum_s w_s O_s / sum_s w_s (bf16), lse = M + ln sum_s w_s. D/8 threads per
// row, 8 columns each, 64 threads per workgroup (decoding has few rows: many
// small workgroups); the split loops are unrolled so that several partials
// are in flight per thread. Rows every split saw no key of get O = 0, lse = -inf.
template <int D>
__global__ __launch_bounds__(64) void fwd_combine_kernel(KvArgs a) {
  constexpr int TPR = D / 8, RPB = 64 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= a.rows) return;
  const int S = a.num_splits;
  const float* pl = a.part_lse + row;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < S; ++s) M = fmaxf(M, pl[(long long)s * a.rows]);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    const float* po = a.part_o + row * D + 8 * part;
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      const float w = __expf(pl[(long long)s * a.rows] - M);  // 0 for splits the row saw no key of
      L += w;
      const float4* p = reinterpret_cast<const float4*>(po + (long long)s * a.rows * D);
      const float4 x0 = p[0], x1 = p[1];
      acc[0] = fmaf(w, x0.x, acc[0]);
      acc[1] = fmaf(w, x0.y, acc[1]);
      acc[2] = fmaf(w, x0.z, acc[2]);
      acc[3] = fmaf(w, x0.w, acc[3]);
      acc[4] = fmaf(w, x1.x, acc[4]);
      acc[5] = fmaf(w, x1.y, acc[5]);
      acc[6] = fmaf(w, x1.z, acc[6]);
      acc[7] = fmaf(w, x1.w, acc[7]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) to_elem(acc[e] * inv, out[e]);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.o) + row * D + 8 * part) = *reinterpret_cast<const uint4*>(out);
  if (part == 0) a.lse[row] = L > 0.f ? M + __logf(L) : -INFINITY;
}

template <int D, int NW, bool CAUSAL>
hipError_t launch_fwd_kv_bf16(const KvArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  // Key blocks of 64, or of 32 for one-wave workgroups (decoding): half the
  // LDS per workgroup, so twice as many workgroups stream K and V per CU.
  constexpr int BN = NW == 1 ? 32 : 64;
  const int G = a.Hq / a.Hkv;
  // Items: row blocks of every (sequence, K/V head); a compact variable-length
  // grid bounds them by the total rows: sum_s ceil(n_s G / BM) <= Tq G / BM + B.
  const long long nrb = a.compact ? ((long long)a.Nq * G + BM - 1) / BM + a.B
                                  : ((long long)a.max_nq * G + BM - 1) / BM * a.B;
  // Linear workgroup ids laid out x-major; 65536 (a multiple of 8) per grid
  // row keeps the XCD of a workgroup that of its linear id.
  const long long total = nrb * a.num_splits * a.Hkv;
  const long long gx = total < 65536 ? total : 65536;
  const long long gy = (total + gx - 1) / gx;
  hipLaunchKernelGGL((fwd_kv_bf16_kernel<D, NW, BN, CAUSAL>), dim3((unsigned)gx, (unsigned)gy), dim3(64 * NW), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  constexpr int RPB = 64 / (D / 8);
  hipLaunchKernelGGL((fwd_combine_kernel<D>), dim3((unsigned)((a.rows + RPB - 1) / RPB)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
