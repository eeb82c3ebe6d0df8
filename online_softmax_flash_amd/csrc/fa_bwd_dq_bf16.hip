// dQ kernel instances of the bf16 backward (see fa_bwd_bf16.hpp). This file is
// compiled with MFMA accumulators in VGPRs (-amdgpu-mfma-vgpr-form): the dQ^T
// accumulator then shares the VGPR file with the scores instead of forcing
// copies through AGPRs, and the kernel stays within two waves per SIMD.
#include "fa_bwd_bf16.hpp"

namespace fa {

template <int D, bool CAUSAL>
static hipError_t dq_bf16(const BwdKvArgs& a, hipStream_t stream) {
  constexpr int NWQ = 4, BM = 32 * NWQ;
  // Compact variable-length grid: sum_s ceil(nq_s / BM) <= Tq / BM + B.
  const long long items = a.compact ? ((long long)a.Nq + BM - 1) / BM + a.B
                                    : (long long)((a.max_nq + BM - 1) / BM) * a.B;
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, NWQ, CAUSAL>), dim3((unsigned)(items * a.Hq)), dim3(64 * NWQ), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream) {
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: return dq_bf16<64, false>(a, stream);
    case 64 * 2 + 1: return dq_bf16<64, true>(a, stream);
    case 128 * 2: return dq_bf16<128, false>(a, stream);
    case 128 * 2 + 1: return dq_bf16<128, true>(a, stream);
    case 256 * 2: return dq_bf16<256, false>(a, stream);
    case 256 * 2 + 1: return dq_bf16<256, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
