// Instances of the general bf16 forward (rectangular, variable length, split keys).
#include "fa_fwd_kv_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t fwd_kv_bf16(const KvArgs& a, int d, int causal, hipStream_t stream) {
  // One wave per workgroup when all packed rows of a (batch, K/V head) fit in
  // 32 (decoding), four otherwise.
  const long long rows = (long long)a.max_nq * (a.Hq / a.Hkv);
  const bool one = rows <= 32;
  // Eight waves (each K/V block staged in LDS then serves 256 rows, half the
  // copies per row) for uniform batches at d = 128 whose row blocks each see
  // 4096 keys or more on average and fill a grid of 4 row blocks or more per
  // (batch, K/V head), with one split: chunked prefill of 2048 queries on
  // 8192 keys 2% faster causal, 9% not causal. Shorter items (a causal square
  // batch of 2048 tokens: 6% slower) and variable-length batches keep four.
  const long long lead = a.max_nk > a.max_nq ? a.max_nk - a.max_nq : 0;
  const long long keys = causal ? lead + (a.max_nq < a.max_nk ? a.max_nq : a.max_nk) / 2 : a.max_nk;
  const bool eight = d == 128 && a.cu_q == nullptr && a.num_splits == 1 && rows >= 1024 && keys >= 4096;
  if (eight) return causal ? launch_fwd_kv_bf16<128, 8, true>(a, stream) : launch_fwd_kv_bf16<128, 8, false>(a, stream);
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
