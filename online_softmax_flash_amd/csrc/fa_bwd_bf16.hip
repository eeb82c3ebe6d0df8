// Instances of the bf16 backward (fa_bwd_bf16.hpp): D and l2, dK and dV, then
// dQ (its instances, and those of the fused dK/dV + dQ launch, are in
// fa_bwd_dq_bf16.hip and fa_bwd_fused_bf16.hip).
#include "fa_bwd_bf16.hpp"

namespace fa {

hipError_t bwd_bf16(const BwdKvArgs& a, int d, int causal, hipStream_t stream) {
  // dK/dV and dQ in one launch (dQ workgroups filling the compute units the
  // dK/dV part's last items leave idle), except where the dK/dV kernel takes
  // its six-pair form (causal d = 128 grids of four or more rounds), which
  // the fused launch's single workgroup size rules out: long_8k 1.79 ms in
  // two launches against 1.85 fused. Fused: wide_4k 2.61 -> 2.48 ms,
  // varlen_mix 1.04 -> 0.98 ms, chunk_2k_8k 0.87 -> 0.84 ms, bwd_4k -2.8%
  // (-1.5% not causal), gqa_4k unchanged.
  const long long wgs6 = (long long)((a.max_nk + 191) / 192) * a.Hkv * a.B;
  const bool six = d == 128 && causal && a.cu_q == nullptr && wgs6 >= 4LL * device_cu_count();
  const bool fused = !six;
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
