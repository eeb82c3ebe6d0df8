// Backward in one pass over the score blocks, bf16 storage: dK, dV and dQ of
// exact softmax attention from a single recomputation of every score block
// (fanfani.net "FlashAttention", section "The backward pass, and where the
// memory saving comes from": the scores are rebuilt from Q, K and the saved
// per-query statistic; synthetic.wiki "FlashAttention: attention's bottleneck
// is the wire, not the maths", section "The backward pass buys memory with
// recompute"). Per (query block, key block) pair the method needs five
// products -- S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q and
// dQ += dS K -- and this kernel issues exactly those five.
//
// Work: one workgroup per (block of 32*NP keys, K/V head, sequence), as in
// bwd_dkdv_bf16_kernel (fa_bwd_bf16.hpp): NP pairs of waves, the P wave of a
// pair holding K and dV^T, its dS wave V and dK^T; Q, dO, lse*log2(e) and
// D = rowsum(dO o O) stream through LDS in double-buffered blocks of 64
// queries, over every query head of the K/V head's group. What is added:
//
//  * The K block also stays in LDS for the whole kernel (the B operand of
//    dQ = dS K, read with transposing reads).
//  * The dS waves write their dS (bf16, the same values dK^T is built from)
//    to an LDS tile whose rows are keys, 16 bytes per lane. At the next step
//    (after the barrier that lands the next query block, so no extra barrier
//    is needed) the dS waves compute the previous step's dQ tile, 64 queries
//    x d over the workgroup's keys, while the P waves take their
//    exponentials, and add it into an fp32 accumulator in the workspace with
//    atomic adds (global_atomic_add_f32: one instruction per accumulator
//    register, a 128-byte row segment per half wave). A last small kernel
//    scales that accumulator and rounds it to bf16.
//  * dQ of a query block is thus summed over key blocks in whatever order
//    the workgroups finish: fp32 addition is not associative, so dQ may
//    differ in its last bits between runs; dK and dV do not.
//
// Shapes: Nq queries and Nk keys per sequence with the causal mask aligned to
// the bottom right (query i sees key j iff j <= i + Nk - Nq), uniform [B, H,
// N, d] batches or variable-length sequences packed along the token axis
// ([H, T, d] with cu_seqlens), as the general forward (fa_fwd_kv_bf16.hpp).
// The square backward is the case Nq = Nk.
#pragma once

#include "fa_bwd_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

// Per query row: D = dO . O and l2 = lse * log2(e), and the row of the dQ
// accumulator cleared; one row per D/8 threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kv_bf16_kernel(BwdKvArgs a) {
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
    float4* z = reinterpret_cast<float4*>(a.dqa + row * D + part * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < a.rows && part == 0) {
    a.dsum[row] = acc;
    a.l2[row] = a.lse[row] * kLog2eF;
  }
}

// dQ = scale * (fp32 accumulator), rounded to bf16; 8 elements per thread.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdKvArgs a) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= a.rows * D) return;
  const float4* s = reinterpret_cast<const float4*>(a.dqa + i);
  const float4 x0 = s[0], x1 = s[1];
  const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  uint16_t out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) to_elem(xs[e] * a.scale, out[e]);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.dq) + i) = *reinterpret_cast<const uint4*>(out);
}

template <int D, int NP, bool CAUSAL>
__global__ __launch_bounds__(128 * NP) void bwd_fused_bf16_kernel(BwdKvArgs a) {
  constexpr int NW = 2 * NP;
  constexpr int BKV = 32 * NP, BQ = 64;
  constexpr int RS = 2 * D + 16;  // padded LDS row bytes of Q, dO and the resident K
  constexpr int NF = D / 16, NDT = D / 32;
  constexpr int TILE = BQ * RS;
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;
  constexpr int PX = 2 * 64 * 16 * 4;  // P exchange bytes per pair: 2 subtiles x 64 lanes x 16 fp32
  constexpr int KRES = BKV * RS;
  constexpr int DSR = 2 * BQ + 16;  // dS tile row (one key): the step's 64 queries in bf16, + padding
  constexpr int OFF_PX = 2 * STAGE, OFF_K = OFF_PX + NP * PX, OFF_DS = OFF_K + KRES;
  constexpr int LDS_BYTES = OFF_DS + BKV * DSR;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one workgroup");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  // The step's dQ tile (2 query subtiles x NDT column tiles of 32) is split
  // over the NP dS waves, TPW column tiles of one subtile each.
  constexpr int NDQ = 2 * NDT;
  constexpr int TPW = NDQ / NP;
  static_assert(NDQ % NP == 0 && NDT % TPW == 0, "dQ tiles split evenly over the dS waves");
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
  decode_block(blockIdx.x, a.Hkv, a.B, nkb_max, false, b, hkv, kb);  // key block 0 has the most work

  // Sequence b: query rows qs .. qs+nq-1, key rows ks .. ks+nk-1 of each head.
  int qs = 0, nq = a.Nq, ks = 0, nk = a.Nk;
  long long q_bs = (long long)a.Hq * a.Nq, q_hs = a.Nq, k_bs = (long long)a.Hkv * a.Nk, k_hs = a.Nk;
  if (a.cu_q != nullptr) {
    // Offsets clamped into [0, total], lengths to the grid's maximum: any
    // offsets keep every access in bounds.
    qs = min(max(a.cu_q[b], 0), a.Nq);
    nq = min(min(max(a.cu_q[b + 1], qs), a.Nq) - qs, a.max_nq);
    ks = min(max(a.cu_k[b], 0), a.Nk);
    nk = min(min(max(a.cu_k[b + 1], ks), a.Nk) - ks, a.max_nk);
    q_bs = 0;
    k_bs = 0;
  }
  const int k0 = kb * BKV;
  if (k0 >= nk || nq <= 0) return;  // uniform over the workgroup: no barrier reached yet
  const int off = CAUSAL ? nk - nq : 0;  // causal: query i sees key j iff j <= i + off
  const int kw0 = k0 + pair * 32;
  const int kj = kw0 + li;  // this lane's key
  const long long krow0 = (long long)b * k_bs + (long long)hkv * k_hs + ks;

  // Steps: (query head g of the group, query block), queries from the first
  // block any key of this workgroup is visible to.
  const int nqb = (nq + BQ - 1) / BQ;
  const int qb_start = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int nqs = max(nqb - qb_start, 0);
  const int nsteps = G * nqs;
  auto qrow0_of = [&](int g) { return (long long)b * q_bs + (long long)(hkv * G + g) * q_hs + qs; };

  BlockDma<D, BQ, RS, NW> dma;
  dma.init(wave, lane);
  auto prefetch = [&](int i) {
    const int g = i / nqs, q0 = (qb_start + i % nqs) * BQ;
    const long long qr = qrow0_of(g);
    uint8_t* st = smem + (i & 1) * STAGE;
    const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + (qr + q0) * D;
    const uint16_t* Og = static_cast<const uint16_t*>(a.dout) + (qr + q0) * D;
    if (q0 + BQ <= nq) {
      dma.template issue<true>(st, Qg, BQ, wave);
      dma.template issue<true>(st + TILE, Og, BQ, wave);
    } else {
      dma.template issue<false>(st, Qg, nq - q0, wave);
      dma.template issue<false>(st + TILE, Og, nq - q0, wave);
    }
    if (wave == 0) dma_row_stats(st + 2 * TILE, a.l2 + qr, q0, nq, lane);
    if (wave == NW - 1) dma_row_stats(st + 2 * TILE + BQ * 4, a.dsum + qr, q0, nq, lane);
  };
  {
    // The K block into LDS once (rows past the sequence read its last key).
    BlockDma<D, BKV, RS, NW> kdma;
    kdma.init(wave, lane);
    const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (krow0 + k0) * D;
    if (k0 + BKV <= nk) kdma.template issue<true>(smem + OFF_K, Kg, BKV, wave);
    else kdma.template issue<false>(smem + OFF_K, Kg, nk - k0, wave);
  }
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
  uint8_t* px = smem + OFF_PX + pair * PX + 16 * lane;
  // dS tile: row = key of the workgroup (pair*32 + li), 16 bytes per
  // (subtile, fragment, lane half). The dQ product reads it transposed: a
  // lane of half h gathers keys 16j + h + 2n + 4e (e = 0..3, n = 0, 1) of
  // one query position -- the key order of the resident K reads below.
  uint8_t* ds_w = smem + OFF_DS + (pair * 32 + li) * DSR + 16 * h;
  const int dq_sub = (pair * TPW) / NDT;      // this dS wave's query subtile of the dQ tile
  const int dq_t0 = (pair * TPW) % NDT;       // and its first column tile
  const uint8_t* ds_r = smem + OFF_DS + (4 * (i16 >> 2) + h) * DSR + 2 * (32 * dq_sub + 16 * (g16 & 1) + 4 * (i16 & 3));
  const uint8_t* k_r = smem + OFF_K + tr_off + 64 * dq_t0;

  // dQ of a finished step (queries q0p.. of the head whose first row is
  // qrp): dS (LDS) times the resident K, added into the fp32 accumulator.
  // Query of accumulator element r of half h: the dS tile's column order
  // (the dS waves' rho row order, kept by their 16-byte writes).
  auto dq_step = [&](long long qrp, int q0p) {
    f32x16 dacc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) dacc[u] = zero16();
#pragma unroll
    for (int j = 0; j < BKV / 16; ++j) {
      const bf16x8 af = tr_frag(ds_r + 16 * j * DSR, 2 * DSR);
#pragma unroll
      for (int u = 0; u < TPW; ++u) mma(dacc[u], af, tr_frag(k_r + 16 * j * RS + 64 * u, 2 * RS));
    }
    const int qsub = q0p + 32 * dq_sub;
    float* dst = a.dqa + (qrp + qsub) * D + 32 * dq_t0 + li;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qo = 16 * (r >> 3) + ((r >> 2) & 1) + 2 * h + 4 * (r & 3);
      if (qsub + qo < nq) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) unsafeAtomicAdd(dst + (long long)qo * D + 32 * u, dacc[u][r]);
      }
    }
  };

  long long qr_prev = 0;
  int q0_prev = 0;
  for (int i = 0; i < nsteps; ++i) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // barrier 1: step i has landed; every wave is done with step i-1; dS of step i-1 visible
    if (i + 1 < nsteps) prefetch(i + 1);
    const int q0 = (qb_start + i % nqs) * BQ;
    const long long qr = qrow0_of(i / nqs);
    const uint8_t* st = smem + (i & 1) * STAGE;
    const float* l2s = reinterpret_cast<const float*>(st + 2 * TILE);
    const float* dss = l2s + BQ;
    // Subtile sub (queries q0 + 32 sub ..) is needed unless it is past nq or
    // (causal) every key of the pair follows every query of it.
    const bool need0 = !CAUSAL || q0 + 31 + off >= kw0;
    const bool need1 = q0 + 32 < nq && (!CAUSAL || q0 + 63 + off >= kw0);
    const uint8_t* qsm = st;
    const uint8_t* osm = st + TILE;
    const uint8_t* rows = pwave ? qsm : osm;
    const uint8_t* trs = pwave ? osm : qsm;
    f32x16 x[2];
    auto products = [&](int sub) {
      x[sub] = zero16();
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(x[sub], *reinterpret_cast<const bf16x8*>(rows + sub * 32 * RS + row_off + 32 * f), kvf[f]);
    };
    bf16x8 bfr[2][2];
    if (!pwave) {
      // The previous step's dQ first: its accumulators are free again before
      // the dP products' are taken.
      if (i > 0) dq_step(qr_prev, q0_prev);
      products(0);
      products(1);
    } else {
      products(0);
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
    // Barrier 2: P visible to the dS waves; every dS wave is done reading dS
    // of step i-1. LDS only: the next step's copies and this step's atomics
    // stay in flight.
    lds_barrier();
    if (!pwave) {
      // dS = P (dP - D) in bf16 fragments, also to the dS tile (zeros for a
      // subtile that is not needed).
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (!(sub ? need1 : need0)) {
          const uint4 z = make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4*>(ds_w + 64 * sub) = z;
          *reinterpret_cast<uint4*>(ds_w + 64 * sub + 32) = z;
          continue;
        }
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
        *reinterpret_cast<bf16x8*>(ds_w + 64 * sub) = bfr[sub][0];
        *reinterpret_cast<bf16x8*>(ds_w + 64 * sub + 32) = bfr[sub][1];
      }
    }
    // acc += tr . bfr (contraction over the 32 queries of each subtile):
    // dV^T += dO^T P (P wave), dK^T += Q^T dS (dS wave).
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (!(sub ? need1 : need0)) continue;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int t = 0; t < NDT; ++t)
          mma(acc[t], tr_frag(trs + sub * 32 * RS + tr_off + 16 * c2 * RS + 64 * t, 2 * RS), bfr[sub][c2]);
    }
    qr_prev = qr;
    q0_prev = q0;
  }
  if (nsteps > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // dS of the last step visible
    if (!pwave) dq_step(qr_prev, q0_prev);
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

template <int D, bool CAUSAL>
hipError_t launch_bwd_fused_bf16(const BwdKvArgs& a, hipStream_t stream) {
  constexpr int NP = 4;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_prep_kv_bf16_kernel<D>), dim3((unsigned)((a.rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     a);
  const int nkb = (a.max_nk + 32 * NP - 1) / (32 * NP);
  hipLaunchKernelGGL((bwd_fused_bf16_kernel<D, NP, CAUSAL>), dim3((unsigned)(nkb * a.Hkv * a.B)), dim3(128 * NP), 0,
                     stream, a);
  const long long n8 = a.rows * D / 8;
  hipLaunchKernelGGL((bwd_dq_convert_kernel<D>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
