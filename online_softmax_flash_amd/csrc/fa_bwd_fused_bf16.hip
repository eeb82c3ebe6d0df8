// Fused dK/dV + dQ instances of the bf16 backward (see fa_bwd_bf16.hpp),
// built with MFMA accumulators in VGPRs like the dQ kernel.
#include "fa_bwd_bf16.hpp"

namespace fa {

template <int D, bool CAUSAL>
static hipError_t fused_bf16(const BwdKvArgs& a, hipStream_t stream) {
  constexpr int NP = D <= 128 ? 4 : 2, NWQ = 2 * NP, BKV = 32 * NP, BM = 32 * NWQ;
  const long long n1 = a.compact ? (((long long)a.Nk + BKV - 1) / BKV + a.B) * a.Hkv
                                 : (long long)((a.max_nk + BKV - 1) / BKV) * a.B * a.Hkv;
  const long long n1p = (n1 + 7) / 8 * 8;
  const long long n2 = a.compact ? (((long long)a.Nq + BM - 1) / BM + a.B) * a.Hq
                                 : (long long)((a.max_nq + BM - 1) / BM) * a.B * a.Hq;
  hipLaunchKernelGGL((bwd_fused_bf16_kernel<D, NP, NWQ, CAUSAL>), dim3((unsigned)(n1p + n2)), dim3(128 * NP), 0,
                     stream, a, (int)n1p);
  return hipGetLastError();
}

hipError_t launch_bwd_fused_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream) {
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: return fused_bf16<64, false>(a, stream);
    case 64 * 2 + 1: return fused_bf16<64, true>(a, stream);
    case 128 * 2: return fused_bf16<128, false>(a, stream);
    case 128 * 2 + 1: return fused_bf16<128, true>(a, stream);
    case 256 * 2: return fused_bf16<256, false>(a, stream);
    case 256 * 2 + 1: return fused_bf16<256, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
