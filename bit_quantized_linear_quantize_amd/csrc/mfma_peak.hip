// Measured peak of the matrix instruction the product kernel uses
// (v_mfma_f32_32x32x16_f16).
//
// One workgroup of 8 waves per CU (two waves per SIMD); every wave issues
// `iters` rounds of 8 independent 32x32x16 f16 products (8 accumulators, so
// no product waits for the previous one); each lane's operands stay the same
// from product to product.  This is a benchmark
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

// The same rate with operands that change from one product to the next, as
// in a matrix product of quantized data: each lane holds four A and four B
// operands whose values are small integers times an fp16 scale (pseudo-random
// from a hash of the lane and position), and consecutive products use
// different pairs, so that the operand bits switch on every instruction.
__device__ __forceinline__ uint32_t peak_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(512) void mfma_f16_peak_switching_kernel(int64_t iters, float* sink) {
  const uint32_t t = blockIdx.x * 512u + threadIdx.x;
  f16x8 a[4], b[4];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = peak_hash(t * 64u + v * 8u + i), hb = peak_hash(~(t * 64u + v * 8u + i));
      // q in [-7, 7] times a scale in [2^-4, 2^-3) (11-bit fp16 values)
      a[v][i] = (_Float16)((float)((int)(ha % 15u) - 7) * (0.0625f + (float)(ha >> 24) * 2.44140625e-4f));
      b[v][i] = (_Float16)((float)((int)(hb % 15u) - 7) * (0.0625f + (float)(hb >> 24) * 2.44140625e-4f));
    }
  f32x16 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[u & 3], b[(u + (u >> 2)) & 3], acc[u], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += acc[u][0] + acc[u][15];
  sink[t] = s;
}

extern "C" {

// As svdq_peak_mfma_f16, with operands that switch on every product.
int svdq_peak_mfma_f16_switching(int64_t iters, int blocks, void* sink, void* stream) {
  hipLaunchKernelGGL(mfma_f16_peak_switching_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters,
                     (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Runs `blocks` workgroups of 512 threads, each wave issuing 8 * iters
// products of 32 x 32 x 16 (32768 flops each).  sink: float [blocks * 512]
// device buffer.  Returns 0, or -5 on a launch error.
int svdq_peak_mfma_f16(int64_t iters, int blocks, void* sink, void* stream) {
  hipLaunchKernelGGL(mfma_f16_peak_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
