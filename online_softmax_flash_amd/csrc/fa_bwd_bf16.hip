// Instances of the bf16 backward (fa_bwd_bf16.hpp): D and l2, dK and dV, then
// dQ (its instances are in fa_bwd_dq_bf16.hip).
#include "fa_bwd_bf16.hpp"

namespace fa {

hipError_t bwd_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream) {
  hipError_t e;
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: e = launch_bwd_prep_dkdv_bf16<64, false>(a, stream); break;
    case 64 * 2 + 1: e = launch_bwd_prep_dkdv_bf16<64, true>(a, stream); break;
    case 128 * 2: e = launch_bwd_prep_dkdv_bf16<128, false>(a, stream); break;
    case 128 * 2 + 1: e = launch_bwd_prep_dkdv_bf16<128, true>(a, stream); break;
    case 256 * 2: e = launch_bwd_prep_dkdv_bf16<256, false>(a, stream); break;
    case 256 * 2 + 1: e = launch_bwd_prep_dkdv_bf16<256, true>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_bwd_dq_bf16(a, d, causal, stream);
}

}  // namespace fa
