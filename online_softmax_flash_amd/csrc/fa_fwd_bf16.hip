// Forward kernel instances, bf16 storage.
#include "fa_fwd.hpp"
#include "fa_fwd_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream) {
  const FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, c};
  // d = 64: 16-wave workgroups (512 rows, four waves per SIMD, 128 registers
  // a wave) on long sequences
  // with a query block of 512 rows for every CU or more: 9-11% faster at
  // N = 2048-8192 than 8 waves, whose softmax work per product is twice that
  // at d = 128; slower on short or few sequences, which keep 8 waves.
  const bool wide64 = N >= 2048 && (long long)((N + 511) / 512) * Hq * B >= device_cu_count();
  switch (d * 2 + (causal ? 1 : 0)) {
    case 64 * 2:
      return wide64 ? launch_fwd_bf16<64, 64, 16, false>(a, stream) : launch_fwd_bf16<64, 64, 8, false>(a, stream);
    case 64 * 2 + 1:
      return wide64 ? launch_fwd_bf16<64, 64, 16, true>(a, stream) : launch_fwd_bf16<64, 64, 8, true>(a, stream);
    case 128 * 2: return launch_fwd_bf16<128, 64, 8, false>(a, stream);
    case 128 * 2 + 1: return launch_fwd_bf16<128, 64, 8, true>(a, stream);
    case 256 * 2: return launch_fwd_bf16<256, 64, 4, false>(a, stream);
    case 256 * 2 + 1: return launch_fwd_bf16<256, 64, 4, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
