// Forward kernel instances, fp32 storage (check mode).
#include "fa_fwd.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream) {
  const FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, c};
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: return launch_fwd<float, 64, 64, false>(a, stream);
    case 64 * 2 + 1: return launch_fwd<float, 64, 64, true>(a, stream);
    case 128 * 2: return launch_fwd<float, 128, 64, false>(a, stream);
    case 128 * 2 + 1: return launch_fwd<float, 128, 64, true>(a, stream);
    case 256 * 2: return launch_fwd<float, 256, 32, false>(a, stream);
    case 256 * 2 + 1: return launch_fwd<float, 256, 32, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
