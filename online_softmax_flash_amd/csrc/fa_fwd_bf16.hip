// Forward kernel instances, bf16 storage.
#include "fa_fwd.hpp"
#include "fa_fwd_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream) {
  const FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, c};
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2: return launch_fwd_bf16<64, 64, 8, false>(a, stream);
    case 64 * 2 + 1: return launch_fwd_bf16<64, 64, 8, true>(a, stream);
    case 128 * 2: return launch_fwd_bf16<128, 64, 8, false>(a, stream);
    case 128 * 2 + 1: return launch_fwd_bf16<128, 64, 8, true>(a, stream);
    case 256 * 2: return launch_fwd_bf16<256, 64, 4, false>(a, stream);
    case 256 * 2 + 1: return launch_fwd_bf16<256, 64, 4, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
