// Measured peak of the matrix instruction the product kernel uses
// (v_mfma_f32_32x32x16_f16).
//
// One workgroup of 8 waves per CU (two waves per SIMD); every wave issues
// `iters` rounds of 8 independent 32x32x16 f16 products (8 accumulators, so
// no product waits for the previous one) on non-constant operands (the
// sustained clock depends on how many bits switch).  This is a benchmark
// helper, built into its own library; it is not part of the layer's
// interface.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void mfma_f16_peak_kernel(int64_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (lane + i));
    b[i] = (_Float16)(0.002f * (lane - i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[u], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += acc[u][0] + acc[u][15];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the products live
}

extern "C" {

// Runs `blocks` workgroups of 512 threads, each wave issuing 8 * iters
// products of 32 x 32 x 16 (32768 flops each).  sink: float [blocks * 512]
// device buffer.  Returns 0, or -5 on a launch error.
int svdq_peak_mfma_f16(int64_t iters, int blocks, void* sink, void* stream) {
  hipLaunchKernelGGL(mfma_f16_peak_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
