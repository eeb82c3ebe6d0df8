// Instances of the bf16 backward (fa_bwd_bf16.hpp): D and l2, dK and dV, then
// dQ (its instances, and those of the fused dK/dV + dQ launch, are in
// fa_bwd_dq_bf16.hip and fa_bwd_fused_bf16.hip).
#include "fa_bwd_bf16.hpp"

namespace fa {

hipError_t bwd_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream) {
  // dK/dV and dQ in one launch (dQ workgroups filling the compute units the
  // dK/dV part's last items leave idle) at d = 256, for variable-length
  // batches and for Nq != Nk: wide_4k 2.61 -> 2.48 ms, varlen_mix 1.04 ->
  // 0.98 ms, chunk_2k_8k 0.87 -> 0.84 ms. Square batches at d <= 128 keep two
  // launches: there the dK/dV kernel's six-pair form, which the fused
  // launch's single workgroup size rules out, or the two smaller kernels
  // measured faster (long_8k 1.82 against 1.94 ms, gqa_4k 3% slower fused).
  const bool fused = d == 256 || a.cu_q != nullptr || a.Nq != a.Nk;
  hipError_t e;
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: e = launch_bwd_prep_dkdv_bf16<64, false>(a, fused, stream); break;
    case 64 * 2 + 1: e = launch_bwd_prep_dkdv_bf16<64, true>(a, fused, stream); break;
    case 128 * 2: e = launch_bwd_prep_dkdv_bf16<128, false>(a, fused, stream); break;
    case 128 * 2 + 1: e = launch_bwd_prep_dkdv_bf16<128, true>(a, fused, stream); break;
    case 256 * 2: e = launch_bwd_prep_dkdv_bf16<256, false>(a, fused, stream); break;
    case 256 * 2 + 1: e = launch_bwd_prep_dkdv_bf16<256, true>(a, fused, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return fused ? launch_bwd_fused_bf16(a, d, causal, stream) : launch_bwd_dq_bf16(a, d, causal, stream);
}

}  // namespace fa
