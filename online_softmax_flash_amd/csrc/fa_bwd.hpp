// Backward kernels: gradients of sum(dO * O) for exact softmax attention,
// recomputing every score block from Q, K and the forward's saved per-query
// statistic lse instead of storing the attention weights (fanfani.net
// "FlashAttention", section "The backward pass, and where the memory saving
// comes from"; synthetic.wiki "FlashAttention: attention's bottleneck is the
// wire, not the maths", section "The backward pass buys memory with
// recompute"). With lse the weights come back in one step, no second pass:
// P_ij = exp(S_ij - lse_i) = exp2(s_ij * c - lse_i * log2(e)).
//
// Chain rule of O = P V, P = softmax(S), S = scale Q K^T:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Three launches on one stream:
//   1. bwd_dot_kernel: D_i = dO_i . O_i (fp32, into the workspace);
//   2. bwd_dkdv_kernel: one workgroup per (key block, K/V head, batch); each
//      wave keeps 32 rows of K and V in registers and accumulates dK and dV
//      over every query head of the group and every query block that sees
//      them -- no atomics, deterministic;
//   3. bwd_dq_kernel: one workgroup per (query block, query head, batch);
//      each wave keeps its 32 query rows of Q and dO in registers and
//      accumulates dQ over the visible key blocks.
// Matrix-core conventions (fragments, sigma row order, C layout) are those of
// fa_device.hpp and the forward kernel.
#pragma once

#include "fa_device.hpp"
#include "fa_fwd.hpp"

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace: D_i, [B, Hq, N]
  int B, Hq, Hkv, N;
  float c;      // scale * log2(e)
  float scale;
};

constexpr float kLog2eF = 1.4426950408889634f;

// D_i = sum_c dO_ic O_ic, one row per D/8 consecutive threads.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const long long rows = (long long)a.B * a.Hq * a.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const T* o = static_cast<const T*>(a.o) + row * D + part * 8;
    const T* g = static_cast<const T*>(a.dout) + row * D + part * 8;
    const typename Elem<T>::frag of = global_frag<T>(o), gf = global_frag<T>(g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)of[e], (float)gf[e], acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) a.dsum[row] = acc;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4, BKV = 32 * NW, NT = 64 * NW, BQ = 32;
  constexpr int NF = D / 16, NDT = D / 32;
  using F = typename Elem<T>::frag;
  using RowTile = SwzTile<BQ, D * sizeof(T)>;  // Q, dO: [BQ][D]
  using TrTile = SwzTile<D, BQ * sizeof(T)>;   // Q^T, dO^T: [D][BQ]
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * RowTile::kBytes + 2 * TrTile::kBytes];
  __shared__ float lse_s[BQ];
  __shared__ float dsum_s[BQ];
  uint8_t* q_s = smem;
  uint8_t* do_s = q_s + RowTile::kBytes;
  uint8_t* qt_s = do_s + RowTile::kBytes;
  uint8_t* dot_s = qt_s + TrTile::kBytes;

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int nkb = (N + BKV - 1) / BKV;
  int b, hkv, kb;
  decode_block(blockIdx.x, a.Hkv, a.B, nkb, false, b, hkv, kb);  // key block 0 has the most work
  const int G = a.Hq / a.Hkv;
  const int k0 = kb * BKV;
  const int kw0 = k0 + wave * 32;
  const int kj = kw0 + li;  // this lane's key row

  const size_t kvoff = (size_t)(b * a.Hkv + hkv) * N * D;
  const T* K = static_cast<const T*>(a.k) + kvoff;
  const T* V = static_cast<const T*>(a.v) + kvoff;
  F kf[NF], vf[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    kf[f] = (kj < N) ? global_frag<T>(K + (size_t)kj * D + 16 * f + 8 * h) : zero_frag<F>();
    vf[f] = (kj < N) ? global_frag<T>(V + (size_t)kj * D + 16 * f + 8 * h) : zero_frag<F>();
  }
  f32x16 dk_acc[NDT], dv_acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dk_acc[t] = zero16();
    dv_acc[t] = zero16();
  }
  const float c = a.c;
  const int nqb = (N + BQ - 1) / BQ;
  const int qb_start = CAUSAL ? k0 / BQ : 0;

  for (int g = 0; g < G; ++g) {
    const int hq = hkv * G + g;
    const size_t qoff = (size_t)(b * a.Hq + hq) * N;
    const T* Q = static_cast<const T*>(a.q) + qoff * D;
    const T* dO = static_cast<const T*>(a.dout) + qoff * D;
    for (int qb = qb_start; qb < nqb; ++qb) {
      const int q0 = qb * BQ;
      __syncthreads();
      stage_rows<T, BQ, D, NT, RowTile>(q_s, Q + (size_t)q0 * D, N - q0, tid);
      stage_rows<T, BQ, D, NT, RowTile>(do_s, dO + (size_t)q0 * D, N - q0, tid);
      stage_rows_transposed<T, BQ, D, NT, TrTile>(qt_s, Q + (size_t)q0 * D, N - q0, tid);
      stage_rows_transposed<T, BQ, D, NT, TrTile>(dot_s, dO + (size_t)q0 * D, N - q0, tid);
      if (tid < BQ) {
        const int qi = q0 + tid;
        // Rows past N get lse = +inf: their weights come out exactly 0.
        lse_s[tid] = (qi < N) ? a.lse[qoff + qi] * kLog2eF : INFINITY;
        dsum_s[tid] = (qi < N) ? a.dsum[qoff + qi] : 0.f;
      }
      __syncthreads();
      if (CAUSAL && q0 + BQ - 1 < kw0) continue;  // every key of this wave is after every query

      // S = Q K^T for this wave's 32 keys: rows = queries (sigma order), columns = keys.
      f32x16 s = zero16();
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(s, lds_frag<T, RowTile>(q_s, sigma(li), 16 * f + 8 * h), kf[f]);
      const bool masked = CAUSAL && q0 < kw0 + 31;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = sigma_row(r, h);
        p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse_s[qr]));
        if (masked && kj > q0 + qr) p[r] = 0.f;
      }
      F pf[2];
      pack_frag(pf[0], p);
      pack_frag(pf[1], p + 8);
      // dV^T += dO^T P
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int t = 0; t < NDT; ++t)
          mma(dv_acc[t], lds_frag<T, TrTile>(dot_s, 32 * t + li, 16 * c2 + 8 * h), pf[c2]);
      // dP = dO V^T
      f32x16 dp = zero16();
#pragma unroll
      for (int f = 0; f < NF; ++f) mma(dp, lds_frag<T, RowTile>(do_s, sigma(li), 16 * f + 8 * h), vf[f]);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dp[r] - dsum_s[sigma_row(r, h)]);
      F dsf[2];
      pack_frag(dsf[0], ds);
      pack_frag(dsf[1], ds + 8);
      // dK^T += Q^T dS
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int t = 0; t < NDT; ++t)
          mma(dk_acc[t], lds_frag<T, TrTile>(qt_s, 32 * t + li, 16 * c2 + 8 * h), dsf[c2]);
    }
  }

  if (kj < N) {
    T* dK = static_cast<T*>(a.dk) + kvoff + (size_t)kj * D;
    T* dV = static_cast<T*>(a.dv) + kvoff + (size_t)kj * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        T ok[4], ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          to_elem(dk_acc[t][4 * gq + e] * a.scale, ok[e]);
          to_elem(dv_acc[t][4 * gq + e], ov[e]);
        }
        const int col = 32 * t + 8 * gq + 4 * h;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(dK + col) = *reinterpret_cast<const uint2*>(ok);
          *reinterpret_cast<uint2*>(dV + col) = *reinterpret_cast<const uint2*>(ov);
        } else {
          *reinterpret_cast<uint4*>(dK + col) = *reinterpret_cast<const uint4*>(ok);
          *reinterpret_cast<uint4*>(dV + col) = *reinterpret_cast<const uint4*>(ov);
        }
      }
  }
}

template <typename T, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = 4, BM = 32 * NW, NT = 64 * NW;
  constexpr int NF = D / 16, NKT = BN / 32, NDT = D / 32, NKC = BN / 16;
  using F = typename Elem<T>::frag;
  using KTile = SwzTile<BN, D * sizeof(T)>;   // K, V: [BN][D]
  using KtTile = SwzTile<D, BN * sizeof(T)>;  // K^T: [D][BN]
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * KTile::kBytes + KtTile::kBytes];
  uint8_t* k_s = smem;
  uint8_t* v_s = k_s + KTile::kBytes;
  uint8_t* kt_s = v_s + KTile::kBytes;

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

  const size_t qoff = (size_t)(b * a.Hq + hq) * N;
  const T* Q = static_cast<const T*>(a.q) + qoff * D;
  const T* dO = static_cast<const T*>(a.dout) + qoff * D;
  const T* K = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + hkv) * N * D;
  const T* V = static_cast<const T*>(a.v) + (size_t)(b * a.Hkv + hkv) * N * D;
  F qf[NF], of[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    qf[f] = (qi < N) ? global_frag<T>(Q + (size_t)qi * D + 16 * f + 8 * h) : zero_frag<F>();
    of[f] = (qi < N) ? global_frag<T>(dO + (size_t)qi * D + 16 * f + 8 * h) : zero_frag<F>();
  }
  const float lsel2 = (qi < N) ? a.lse[qoff + qi] * kLog2eF : INFINITY;
  const float Di = (qi < N) ? a.dsum[qoff + qi] : 0.f;
  f32x16 dq_acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) dq_acc[t] = zero16();
  const float c = a.c;

  const int nkb = (N + BN - 1) / BN;
  const int q_last = min(q0 + BM, N) - 1;
  const int kb_end = CAUSAL ? min(nkb, q_last / BN + 1) : nkb;
  for (int kb = 0; kb < kb_end; ++kb) {
    const int k0 = kb * BN;
    __syncthreads();
    stage_rows<T, BN, D, NT, KTile>(k_s, K + (size_t)k0 * D, N - k0, tid);
    stage_rows<T, BN, D, NT, KTile>(v_s, V + (size_t)k0 * D, N - k0, tid);
    stage_rows_transposed<T, BN, D, NT, KtTile>(kt_s, K + (size_t)k0 * D, N - k0, tid);
    __syncthreads();
    if (CAUSAL && k0 > qw0 + 31) continue;  // every key of the block is after every query of this wave

    const bool masked = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw0);
    F dsf[NKC];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      // S^T and dP^T = V dO^T for 32 keys (sigma order) x this wave's queries.
      f32x16 s = zero16(), dp = zero16();
      const int krow = 32 * kt + sigma(li);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        mma(s, lds_frag<T, KTile>(k_s, krow, 16 * f + 8 * h), qf[f]);
        mma(dp, lds_frag<T, KTile>(v_s, krow, 16 * f + 8 * h), of[f]);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lsel2));
        if (masked) {
          const int key = k0 + 32 * kt + sigma_row(r, h);
          if (key >= N || (CAUSAL && key > qi)) p = 0.f;
        }
        ds[r] = p * (dp[r] - Di);
      }
      pack_frag(dsf[2 * kt], ds);
      pack_frag(dsf[2 * kt + 1], ds + 8);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int t = 0; t < NDT; ++t)
        mma(dq_acc[t], lds_frag<T, KtTile>(kt_s, 32 * t + li, 16 * kc + 8 * h), dsf[kc]);
  }

  if (qi < N) {
    T* dQ = static_cast<T*>(a.dq) + (qoff + qi) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        T out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(dq_acc[t][4 * gq + e] * a.scale, out[e]);
        const int col = 32 * t + 8 * gq + 4 * h;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(dQ + col) = *reinterpret_cast<const uint2*>(out);
        } else {
          *reinterpret_cast<uint4*>(dQ + col) = *reinterpret_cast<const uint4*>(out);
        }
      }
  }
}

template <typename T, int D, int BN, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_dot_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, a);
  const int nkb = (a.N + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3((unsigned)(nkb * a.Hkv * a.B)), dim3(256), 0, stream, a);
  const int nqb = (a.N + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, BN, CAUSAL>), dim3((unsigned)(nqb * a.Hq * a.B)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
