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
    // d = 256: K, V and both accumulators of 32 keys do not fit one wave's
    // registers next to the working set; the generic kernels serve it.
    case 256 * 2: return launch_bwd<uint16_t, 256, 64, false>(a, stream);
    case 256 * 2 + 1: return launch_bwd<uint16_t, 256, 64, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
