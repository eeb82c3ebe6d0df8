// Backward kernel instances, bf16 storage.
#include "fa_bwd_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* dsum,
                  int B, int Hq, int Hkv, int N, int d, float scale, float c, int causal, hipStream_t stream) {
  const BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, dsum, B, Hq, Hkv, N, c, scale};
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: return launch_bwd_bf16<64, false>(a, stream);
    case 64 * 2 + 1: return launch_bwd_bf16<64, true>(a, stream);
    case 128 * 2: return launch_bwd_bf16<128, false>(a, stream);
    case 128 * 2 + 1: return launch_bwd_bf16<128, true>(a, stream);
    case 256 * 2: return launch_bwd_bf16<256, false>(a, stream);
    case 256 * 2 + 1: return launch_bwd_bf16<256, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
