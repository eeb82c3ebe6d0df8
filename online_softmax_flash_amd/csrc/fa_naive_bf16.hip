// Instances of the three-pass materialising baseline (bf16 storage).
#include "fa_naive_bf16.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t naive_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* s, uint16_t* p,
                      int B, int Hq, int Hkv, int N, int d, float scale, int causal, hipStream_t stream) {
  const NaiveArgs a{q, k, v, o, lse, s, p, B, Hq, Hkv, N, scale, causal};
  switch (d) {
    case 64: return launch_naive_bf16<64>(a, stream);
    case 128: return launch_naive_bf16<128>(a, stream);
    case 256: return launch_naive_bf16<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
