// Forward kernel: exact softmax attention by the online softmax, one
// workgroup per (query block, query head, batch).
//
// The recurrence is that of fanfani.net "FlashAttention", section "A pinch of
// math: making the softmax work in pieces": per query row a running maximum
// m, a running sum of exponentials l and a running weighted sum of values o;
// each key block raises m to max(m, block max), rescales l and o by
// exp(m_old - m_new) (at most 1) and adds the block's exponentials and
// exponential-weighted values; o is divided by l once at the end. The tiling
// (a block of queries against one block of keys and values at a time, the
// score block never leaving the chip) is that of section "Do not materialize
// the matrix".
//
// Mapping onto gfx950:
//  * 4 wavefronts x 32 query rows; the wave's Q rows live in registers as the
//    B operand of S^T = K Q^T, so that each lane owns one query (column) and
//    the row max / row sum of the softmax are in-lane reductions plus one
//    exchange between the two lane halves.
//  * The K block is staged in LDS row-major and read as the A operand with
//    its rows in sigma order; the V block is staged transposed (V^T) and read
//    as the A operand of O^T = V^T P^T. With the sigma row order the
//    probabilities a lane holds are directly its B-operand fragments.
//  * exp2 with the scale folded into log2(e): scores are kept unscaled and
//    exp2(s*c - m) is one FMA and one v_exp_f32, c = scale*log2(e).
//  * Causal: key blocks entirely above the diagonal are never loaded; blocks
//    on the diagonal (and the ragged tail at N) are masked element-wise.
//  * Work order: longest causal query blocks first; all query blocks of a
//    (batch, K/V head) go to one XCD so its K/V stay in that XCD's L2.
#pragma once

#include "fa_device.hpp"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;
  float c;  // scale * log2(e)
};

// Decode a workgroup id into (batch, query head, query block). Workgroups are
// dispatched round-robin over the 8 XCDs; ids are remapped so that each XCD
// receives a contiguous range of (batch, head) pairs, and query blocks are
// issued from the last (longest, when causal) to the first.
__device__ __forceinline__ void decode_block(int wg, int Hq, int B, int nqb, bool causal,
                                             int& b, int& hq, int& qb) {
  const int HB = Hq * B;
  const int level = wg / HB, wp = wg % HB;
  const int p = (HB % 8 == 0) ? ((wp % 8) * (HB / 8) + wp / 8) : wp;
  b = p / Hq;
  hq = p % Hq;
  qb = causal ? (nqb - 1 - level) : level;
}

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  constexpr int NW = 4, BM = 32 * NW, NT = 64 * NW;
  constexpr int NF = D / 16;   // contraction fragments of Q K^T
  constexpr int NKT = BN / 32; // 32-key score tiles per block
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  constexpr int NKC = BN / 16; // 16-key contraction fragments of V^T P^T
  using F = typename Elem<T>::frag;
  using KTile = SwzTile<BN, D * sizeof(T)>;
  using VTile = SwzTile<D, BN * sizeof(T)>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[KTile::kBytes + VTile::kBytes];
  uint8_t* ks = smem;
  uint8_t* vts = smem + KTile::kBytes;

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int nqb = (N + BM - 1) / BM;
  int b, hq, qb;
  decode_block(blockIdx.x, a.Hq, a.B, nqb, CAUSAL, b, hq, qb);
  const int hkv = hq / (a.Hq / a.Hkv);
  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + li;

  const T* Q = static_cast<const T*>(a.q) + (size_t)(b * a.Hq + hq) * N * D;
  const T* K = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + hkv) * N * D;
  const T* V = static_cast<const T*>(a.v) + (size_t)(b * a.Hkv + hkv) * N * D;

  // This lane's query row as B-operand fragments (d = 16f + 8h .. +7).
  F qf[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    qf[f] = (qi < N) ? global_frag<T>(Q + (size_t)qi * D + 16 * f + 8 * h) : zero_frag<F>();

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = zero16();
  float m_run = -INFINITY;  // running max of s*c (log2 units)
  float l_run = 0.f;        // this lane's share of the running denominator
  const float c = a.c;

  const int nkb = (N + BN - 1) / BN;
  const int q_last = min(q0 + BM, N) - 1;
  const int kb_end = CAUSAL ? min(nkb, q_last / BN + 1) : nkb;

  for (int kb = 0; kb < kb_end; ++kb) {
    const int k0 = kb * BN;
    __syncthreads();
    stage_rows<T, BN, D, NT, KTile>(ks, K + (size_t)k0 * D, N - k0, tid);
    stage_rows_transposed<T, BN, D, NT, VTile>(vts, V + (size_t)k0 * D, N - k0, tid);
    __syncthreads();

    // S^T block: rows = keys (sigma order within each 32), columns = this wave's queries.
    f32x16 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      s[kt] = zero16();
      const int krow = 32 * kt + sigma(li);
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(s[kt], lds_frag<T, KTile>(ks, krow, 16 * f + 8 * h), qf[f]);
    }

    const bool masked = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw0);
    if (masked) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kt + sigma_row(r, h);
          if (key >= N || (CAUSAL && key > qi)) s[kt][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxc = (mx == -INFINITY) ? -INFINITY : mx * c;
    const float m_new = fmaxf(m_run, mxc);
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - base);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -base));
        if (masked && s[kt][r] == -INFINITY) p = 0.f;
        s[kt][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;

    // P^T as B-operand fragments: fragment kc holds keys 16kc + 8h .. +7.
    F pf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      float tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = s[kc >> 1][8 * (kc & 1) + e];
      pack_frag(pf[kc], tmp);
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int t = 0; t < NDT; ++t)
        mma(oacc[t], lds_frag<T, VTile>(vts, 32 * t + li, 16 * kc + 8 * h), pf[kc]);
  }

  // Epilogue: divide by the denominator once; lse in natural-log units.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (qi < N) {
    T* O = static_cast<T*>(a.o) + (size_t)(b * a.Hq + hq) * N * D + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(oacc[t][4 * g + e] * inv, out[e]);
        T* dst = O + 32 * t + 8 * g + 4 * h;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(out);
        } else {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(out);
        }
      }
    if (h == 0) a.lse[(size_t)(b * a.Hq + hq) * N + qi] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <typename T, int D, int BN, bool CAUSAL>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 128;
  const int nqb = (a.N + BM - 1) / BM;
  const dim3 grid((unsigned)(nqb * a.Hq * a.B));
  hipLaunchKernelGGL((fwd_kernel<T, D, BN, CAUSAL>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
