// Matrix-core throughput probe, for the roofline of the benchmark: the rate
// the chip reaches on back-to-back v_mfma_f32_32x32x16_bf16 (the product the
// attention kernels use), next to the published dense bf16 peak. Not part of
// the attention library: bench.py loads it on its own.
//
// Every wave runs four independent accumulation chains of `iters` products
// each (operands in registers, no memory traffic in the loop); 1024
// workgroups of 4 waves keep every SIMD of the chip busy. Flops per launch:
// blocks * 4 waves * 4 chains * iters * 2*32*32*16.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(lane * 0.001f + e);
    b[e] = (__bf16)(e * 0.5f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) r += c0[e] + c1[e] + c2[e] + c3[e];
  out[blockIdx.x * 256 + threadIdx.x] = r;  // keeps the products live
}

}  // namespace

// out: device buffer of blocks*256 floats (overwritten). Returns the launch status.
extern "C" int fa_probe_mfma_bf16(float* out, int iters, int blocks, hipStream_t stream) {
  if (out == nullptr || iters <= 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}
