// Instances of the general bf16 forward (rectangular, variable length, split keys).
#include "fa_fwd_kv_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t fwd_kv_bf16(const KvArgs& a, int d, int causal, hipStream_t stream) {
  // One wave per workgroup when all packed rows of a (batch, K/V head) fit in
  // 32 (decoding), four otherwise.
  const bool one = (long long)a.max_nq * (a.Hq / a.Hkv) <= 32;
  switch (d * 4 + (one ? 2 : 0) + (causal ? 1 : 0)) {
    case 64 * 4 + 0: return launch_fwd_kv_bf16<64, 4, false>(a, stream);
    case 64 * 4 + 1: return launch_fwd_kv_bf16<64, 4, true>(a, stream);
    case 64 * 4 + 2: return launch_fwd_kv_bf16<64, 1, false>(a, stream);
    case 64 * 4 + 3: return launch_fwd_kv_bf16<64, 1, true>(a, stream);
    case 128 * 4 + 0: return launch_fwd_kv_bf16<128, 4, false>(a, stream);
    case 128 * 4 + 1: return launch_fwd_kv_bf16<128, 4, true>(a, stream);
    case 128 * 4 + 2: return launch_fwd_kv_bf16<128, 1, false>(a, stream);
    case 128 * 4 + 3: return launch_fwd_kv_bf16<128, 1, true>(a, stream);
    case 256 * 4 + 0: return launch_fwd_kv_bf16<256, 4, false>(a, stream);
    case 256 * 4 + 1: return launch_fwd_kv_bf16<256, 4, true>(a, stream);
    case 256 * 4 + 2: return launch_fwd_kv_bf16<256, 1, false>(a, stream);
    case 256 * 4 + 3: return launch_fwd_kv_bf16<256, 1, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
