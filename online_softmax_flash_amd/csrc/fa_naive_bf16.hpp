// Standard (materialising) attention in three passes through device memory:
// the baseline the online-softmax method removes (fanfani.net
// "FlashAttention", section "The bottleneck was never the arithmetic": the
// score matrix is written out, read back for the mask and the softmax, the
// weights written out and read back for the product with V). It computes
// the same O and lse as the fused forward and exists to measure the HBM
// traffic and time that the fusion saves on the same chip.
//
//   1. naive_scores_kernel:  S = scale * Q K^T for every (query, key) pair,
//      fp32, to the workspace (B*Hq*N*N*4 bytes; causal pairs are computed too);
//   2. naive_softmax_kernel: per row, mask, max, exponentials, sum;
//      P = exp(S - m) / l rounded to bf16 into the workspace, lse = m + ln l;
//   3. naive_pv_kernel:      O = P V, fp32 accumulation, bf16 out.
// The matrix products use the same matrix-core tiles as the fused kernels
// (K and V blocks staged in LDS by direct loads, Q rows and P rows as
// B-operand fragments from global memory).
#pragma once

#include "fa_fwd_bf16.hpp"

namespace fa {

struct NaiveArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* s;     // [B, Hq, N, N] fp32
  uint16_t* p;  // [B, Hq, N, N] bf16
  int B, Hq, Hkv, N;
  float scale;
  int causal;
};

// S^T = K Q^T over every key block, scaled, stored row-major as S[query][key].
template <int D>
__global__ __launch_bounds__(256) void naive_scores_kernel(NaiveArgs a) {
  constexpr int NW = 4, BN = 64;
  using C = Bf16FwdCfg<D, BN, NW>;
  constexpr int NF = D / 16, NKT = BN / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::KBYTES];
  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int nqb = (N + C::BM - 1) / C::BM;
  const int qb = blockIdx.x % nqb, bh = blockIdx.x / nqb;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  const int qi = qb * C::BM + wave * 32 + li;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + (size_t)bh * N * D;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + (size_t)(b * a.Hkv + hkv) * N * D;
  float* S = a.s + ((size_t)bh * N + qi) * N;

  BlockDma<D, BN, C::KROW, NW> dma;
  dma.init(wave, lane);
  const int nkb = (N + BN - 1) / BN;
  auto prefetch = [&](int kb) {
    const int valid = N - kb * BN;
    if (valid >= BN) dma.template issue<true>(smem + (kb & 1) * C::KBYTES, K + (size_t)kb * BN * D, BN, wave);
    else dma.template issue<false>(smem + (kb & 1) * C::KBYTES, K + (size_t)kb * BN * D, valid, wave);
  };
  prefetch(0);
  bf16x8 qf[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    qf[f] = (qi < N) ? global_frag<uint16_t>(Q + (size_t)qi * D + 16 * f + 8 * h) : zero_frag<bf16x8>();
  const int k_off = sigma(li) * C::KROW + 16 * h;
  for (int kb = 0; kb < nkb; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < nkb) prefetch(kb + 1);
    const uint8_t* st = smem + (kb & 1) * C::KBYTES;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      f32x16 s = zero16();
#pragma unroll
      for (int f = 0; f < NF; ++f)
        mma(s, *reinterpret_cast<const bf16x8*>(st + k_off + 32 * kt * C::KROW + 32 * f), qf[f]);
      // Element r of this lane is key k0 + 16*(r/8) + 8h + r%8 of query qi.
      const int k0 = kb * BN + 32 * kt;
      if (qi < N) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int key = k0 + 16 * half + 8 * h;
          if (key + 8 <= N) {
            float4 x0, x1;
            x0.x = s[8 * half + 0] * a.scale;
            x0.y = s[8 * half + 1] * a.scale;
            x0.z = s[8 * half + 2] * a.scale;
            x0.w = s[8 * half + 3] * a.scale;
            x1.x = s[8 * half + 4] * a.scale;
            x1.y = s[8 * half + 5] * a.scale;
            x1.z = s[8 * half + 6] * a.scale;
            x1.w = s[8 * half + 7] * a.scale;
            *reinterpret_cast<float4*>(S + key) = x0;
            *reinterpret_cast<float4*>(S + key + 4) = x1;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key + e < N) S[key + e] = s[8 * half + e] * a.scale;
          }
        }
      }
    }
  }
}

// One workgroup of 256 threads per row: mask, max, sum, P (bf16), lse. Rows
// of up to 256*4*MAXC scores whose length is a multiple of 4 are read once,
// as float4, into registers; other rows are read twice with scalar loads.
constexpr int kNaiveMaxC = 16;

__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = is_max ? fmaxf(x, __shfl_xor(x, o)) : x + __shfl_xor(x, o);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void naive_softmax_kernel(NaiveArgs a) {
  __shared__ float red[4];
  const size_t rowid = blockIdx.x;
  const int N = a.N;
  const int qi = (int)(rowid % N);
  const float* S = a.s + rowid * N;
  uint16_t* P = a.p + rowid * N;
  const int lim = a.causal ? qi : N - 1;  // last visible key
  const int tid = threadIdx.x;
  if (N % 4 == 0 && N <= 1024 * kNaiveMaxC) {
    float4 x[kNaiveMaxC];
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kNaiveMaxC; ++t) {
      const int j = 4 * (tid + 256 * t);
      x[t] = j < N ? *reinterpret_cast<const float4*>(S + j) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (j + 0 > lim) x[t].x = -INFINITY;
      if (j + 1 > lim) x[t].y = -INFINITY;
      if (j + 2 > lim) x[t].z = -INFINITY;
      if (j + 3 > lim) x[t].w = -INFINITY;
      m = fmaxf(m, fmaxf(fmaxf(x[t].x, x[t].y), fmaxf(x[t].z, x[t].w)));
    }
    m = block_reduce(m, true, red);
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < kNaiveMaxC; ++t) {
      x[t].x = __expf(x[t].x - m);
      x[t].y = __expf(x[t].y - m);
      x[t].z = __expf(x[t].z - m);
      x[t].w = __expf(x[t].w - m);
      l += (x[t].x + x[t].y) + (x[t].z + x[t].w);
    }
    l = block_reduce(l, false, red);
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < kNaiveMaxC; ++t) {
      const int j = 4 * (tid + 256 * t);
      if (j < N) {
        uint16_t o4[4] = {__builtin_bit_cast(uint16_t, (__bf16)(x[t].x * inv)),
                          __builtin_bit_cast(uint16_t, (__bf16)(x[t].y * inv)),
                          __builtin_bit_cast(uint16_t, (__bf16)(x[t].z * inv)),
                          __builtin_bit_cast(uint16_t, (__bf16)(x[t].w * inv))};
        *reinterpret_cast<uint2*>(P + j) = *reinterpret_cast<const uint2*>(o4);
      }
    }
    if (tid == 0) a.lse[rowid] = m + __logf(l);
    return;
  }
  float m = -INFINITY;
  for (int j = tid; j <= lim; j += 256) m = fmaxf(m, S[j]);
  m = block_reduce(m, true, red);
  float l = 0.f;
  for (int j = tid; j <= lim; j += 256) l += __expf(S[j] - m);
  l = block_reduce(l, false, red);
  const float inv = 1.f / l;
  for (int j = tid; j < N; j += 256) {
    const float pv = j <= lim ? __expf(S[j] - m) * inv : 0.f;
    P[j] = __builtin_bit_cast(uint16_t, (__bf16)pv);
  }
  if (tid == 0) a.lse[rowid] = m + __logf(l);
}

// O^T = V^T P^T: each wave 32 queries, P rows as B-operand fragments from
// global memory, V blocks staged in LDS and read with transposing reads.
template <int D>
__global__ __launch_bounds__(256) void naive_pv_kernel(NaiveArgs a) {
  constexpr int NW = 4, BN = 64;
  using C = Bf16FwdCfg<D, BN, NW>;
  constexpr int NDT = D / 32, NKC = BN / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::VBYTES];
  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int nqb = (N + C::BM - 1) / C::BM;
  const int qb = blockIdx.x % nqb, bh = blockIdx.x / nqb;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  const int qi = qb * C::BM + wave * 32 + li;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + (size_t)(b * a.Hkv + hkv) * N * D;
  const uint16_t* P = a.p + ((size_t)bh * N + (qi < N ? qi : N - 1)) * N;

  BlockDma<D, BN, C::VROW, NW> dma;
  dma.init(wave, lane);
  const int nkb = (N + BN - 1) / BN;
  auto prefetch = [&](int kb) {
    const int valid = N - kb * BN;
    if (valid >= BN) dma.template issue<true>(smem + (kb & 1) * C::VBYTES, V + (size_t)kb * BN * D, BN, wave);
    else dma.template issue<false>(smem + (kb & 1) * C::VBYTES, V + (size_t)kb * BN * D, valid, wave);
  };
  prefetch(0);
  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = zero16();
  const int v_off = (8 * h + (i16 >> 2)) * C::VROW + 2 * (16 * (g16 & 1) + 4 * (i16 & 3));
  for (int kb = 0; kb < nkb; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < nkb) prefetch(kb + 1);
    const uint32_t vaddr = lds_addr(smem + (kb & 1) * C::VBYTES) + (uint32_t)v_off;
    TrReads<NDT> vr;
    static_for<0, NKC>([&](auto kcc) {
      constexpr int kc = decltype(kcc)::value;
      // Keys k0 + 16kc + 8h .. +7 of this lane's query; keys >= N have P = 0
      // (the rows of V past N in LDS are copies of row N-1).
      const int key = kb * BN + 16 * kc + 8 * h;
      bf16x8 pf;
      if (key + 8 <= N) {
        pf = global_frag<uint16_t>(P + key);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = key + e < N ? __builtin_bit_cast(__bf16, P[key + e]) : (__bf16)0.f;
      }
      vr.template issue<16 * kc * C::VROW, C::VROW>(vaddr);
      vr.template wait<0>();
#pragma unroll
      for (int t = 0; t < NDT; ++t) mma(oacc[t], vr.frag(t), pf);
    });
  }
  if (qi < N) {
    uint16_t* O = static_cast<uint16_t*>(a.o) + ((size_t)bh * N + qi) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint16_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) to_elem(oacc[t][4 * gq + e], out[e]);
        *reinterpret_cast<uint2*>(O + 32 * t + 8 * gq + 4 * h) = *reinterpret_cast<const uint2*>(out);
      }
  }
}

template <int D>
hipError_t launch_naive_bf16(const NaiveArgs& a, hipStream_t stream) {
  const int nqb = (a.N + 127) / 128;
  const unsigned grid = (unsigned)(nqb * a.Hq * a.B);
  hipLaunchKernelGGL((naive_scores_kernel<D>), dim3(grid), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(naive_softmax_kernel, dim3((unsigned)((size_t)a.B * a.Hq * a.N)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((naive_pv_kernel<D>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
