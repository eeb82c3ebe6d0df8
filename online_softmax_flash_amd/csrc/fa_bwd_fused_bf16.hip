// Instances of the one-pass bf16 backward (fa_bwd_fused_bf16.hpp).
#include "fa_bwd_fused_bf16.hpp"

namespace fa {

hipError_t bwd_fused_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream) {
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: return launch_bwd_fused_bf16<64, false>(a, stream);
    case 64 * 2 + 1: return launch_bwd_fused_bf16<64, true>(a, stream);
    case 128 * 2: return launch_bwd_fused_bf16<128, false>(a, stream);
    case 128 * 2 + 1: return launch_bwd_fused_bf16<128, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
