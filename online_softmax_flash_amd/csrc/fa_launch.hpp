// Host-side launchers of the attention kernels (one per storage type).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs;

// Forward: picks the kernel instance for (d, causal) and launches it on stream.
hipError_t fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream);
hipError_t fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float c, int causal, hipStream_t stream);

// Backward: D = rowsum(dO * O) into dsum, then the dK/dV and dQ kernels,
// all on stream.
hipError_t bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* dsum,
                    int B, int Hq, int Hkv, int N, int d, float scale, float c, int causal, hipStream_t stream);
hipError_t bwd_f32(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* dsum,
                   int B, int Hq, int Hkv, int N, int d, float scale, float c, int causal, hipStream_t stream);

}  // namespace fa
