// Measured peaks of the matrix instructions the product kernel uses
// (v_mfma_f32_32x32x16_f16; the int4 inner loop of f8f6f4 products with
// scale products from a bf16 instruction).
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

// An earlier form of the int4 x int4 group products' inner loop: the
// codes (|q| <= 7) are exact fp8 E4M3 or fp6 E2M3 operands, one
// 32x32x64 f8f6f4 product gives a group's integer sum P (64 = the group
// size), and the bf16 group scales, which these instructions cannot take
// (their block scales are powers of two per 32 values), are applied on the
// vector ALU: acc += P * (s_x[row] * s_w[col]), 16 multiplies and 16 FMAs
// per 32x32 tile and group (the same per tile for any wave tile).  A wave
// computes a 64 x 64 block (2 x 2 tiles); its operand pairs rotate and the
// scales change every group.  FMT: 0 = fp8 E4M3, 2 = fp6 E2M3.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int FMT>
__global__ __launch_bounds__(512) void group_scaled_probe_kernel(int64_t iters, float* sink) {
  const uint32_t t = blockIdx.x * 512u + threadIdx.x;
  i32x8 a[2], b[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // bytes of small-magnitude codes (E4M3 / E2M3 patterns of values <= 7)
    const uint32_t h0 = peak_hash(t * 97u + i), h1 = peak_hash(~(t * 89u + i));
    a[0][i] = (int)(h0 & 0x2d3d2d3du);
    a[1][i] = (int)(h1 & 0x3d2d3d2du);
    b[0][i] = (int)((h0 >> 3) & 0x2d3d2d3du);
    b[1][i] = (int)((h1 >> 3) & 0x3d2d3d2du);
  }
  f32x16 sx[2];
  float sw[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sx[0][e] = 0.01f + 1e-4f * (float)((t + e) & 63);
    sx[1][e] = 0.02f + 1e-4f * (float)((t + 3 * e) & 63);
  }
  for (int j = 0; j < 2; ++j) sw[j] = 0.03f + 1e-4f * (float)((t >> j) & 31);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const f32x16 zero = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {  // two groups per iteration with the operand pairs rotated
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(i + v) & 1], b[(j + v) & 1], zero, FMT,
                                                                           FMT, 0, 0x7f, 0, 0x7f);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(p[e], sx[i][e] * sw[j], acc[i][j][e]);
        }
#pragma unroll
      for (int j = 0; j < 2; ++j) sw[j] = sw[j] * 1.0000001f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) s += acc[i][j][0] + acc[i][j][15];
  sink[t] = s;
}

// The int4 product kernel's inner loop as it is built: per 32 x 32 tile and
// group one f8f6f4 product P (codes as fp8 or fp6), one bf16 outer-product
// instruction of K = 8 for the scale products s_x s_w (element 0 of each
// lane's four values the scale, the rest zero), and acc += P * (s_x s_w), 16
// FMAs.  A wave computes a 64 x 96 block (2 x 3 tiles), the kernel's wave
// tile; its operands are marked as changing every group.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int FMT>
__global__ __launch_bounds__(512) void outer_scaled_probe_kernel(int64_t iters, float* sink) {
  const uint32_t t = blockIdx.x * 512u + threadIdx.x;
  i32x8 a[2], b[3];
  uint32_t as[2], bs[3];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h0 = peak_hash(t * 97u + i), h1 = peak_hash(~(t * 89u + i));
    a[0][i] = (int)(h0 & 0x2d3d2d3du);
    a[1][i] = (int)(h1 & 0x3d2d3d2du);
    b[0][i] = (int)((h0 >> 3) & 0x2d3d2d3du);
    b[1][i] = (int)((h1 >> 3) & 0x3d2d3d2du);
    b[2][i] = (int)((h0 >> 5) & 0x3d2d2d3du);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) as[i] = 0x3c00u + (peak_hash(t + 7u * i) & 0x7fu);  // bf16 bits of ~2^-7
#pragma unroll
  for (int j = 0; j < 3; ++j) bs[j] = 0x3c80u + (peak_hash(t + 11u * j) & 0x7fu);
  f32x16 acc[2][3];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const f32x16 zero = {};
  for (int64_t it = 0; it < iters; ++it) {
    // (the compiler may not keep the operands from one group to the next)
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(a[i]), "+v"(as[i]));
#pragma unroll
    for (int j = 0; j < 3; ++j) asm volatile("" : "+v"(b[j]), "+v"(bs[j]));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], zero, FMT, FMT, 0, 0x7f, 0, 0x7f);
        const f32x16 sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4, u32x2{as[i], 0u}),
                                                                   __builtin_bit_cast(s16x4, u32x2{bs[j], 0u}), zero,
                                                                   0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(p[e], sc[e], acc[i][j][e]);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) s += acc[i][j][0] + acc[i][j][15];
  sink[t] = s;
}

extern "C" {

// The product kernel's inner loop above: `iters` groups per wave (6
// products of 32 x 32 x 64, 131072 flops each).  fmt 0: fp8 operands, 2:
// fp6.  Returns 0, -5 on a launch error, -1 on another fmt.
int svdq_peak_outer_scaled(int fmt, int64_t iters, int blocks, void* sink, void* stream) {
  if (fmt == 0)
    hipLaunchKernelGGL(outer_scaled_probe_kernel<0>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters,
                       (float*)sink);
  else if (fmt == 2)
    hipLaunchKernelGGL(outer_scaled_probe_kernel<2>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters,
                       (float*)sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// The group-scaled int4 product loop above: `iters` rounds of two groups per
// wave (8 products of 32 x 32 x 64, 131072 flops each).  fmt 0: fp8
// operands, 2: fp6.  Returns 0, -5 on a launch error, -1 on another fmt.
int svdq_peak_group_scaled(int fmt, int64_t iters, int blocks, void* sink, void* stream) {
  if (fmt == 0)
    hipLaunchKernelGGL(group_scaled_probe_kernel<0>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters,
                       (float*)sink);
  else if (fmt == 2)
    hipLaunchKernelGGL(group_scaled_probe_kernel<2>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters,
                       (float*)sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

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
