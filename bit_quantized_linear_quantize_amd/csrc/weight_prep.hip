// Offline weight preparation on the GPU: the smoothing factors and the
// quantization and packing of the residual weight (what the diffuse-compressor
// tool of the Nunchaku Lite pages does offline before a checkpoint is saved;
// "Resources" section and the "Supported quantization types" table).
//
// Both produce exactly the oracle's bits: the same IEEE operations, in the
// same precision, in the same order for every decision.
//   smooth[k] = bf16_rne(sqrt(amax_m |x[m, k]| / amax_n |w[n, k]|)), ratio and
//     root in fp64, 1 where the result is not finite or not positive;
//   int4:  s = bf16(fl32(amax / 7)), q = rne(fl32(r * fl32(1 / s))), |q| <= 7,
//          sign-magnitude nibbles;
//   nvfp4: t = fl32(amax_tensor / 2688), s8 = E4M3(fl32(amax / fl32(6 t))),
//          S = fl32(dec(s8) t), code = E2M1(fl32(r * fl32(1 / S)));
//   groups with amax < 2^-100 (or a zero scale): scale 0, codes 0.
// The low-rank split between the two (an SVD of the smoothed weight) is in
// prep_svd.hip.
//
// Column maxima and the tensor maximum are reduced with atomicMax on the bit
// patterns of non-negative floats, whose order is that of the values.

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

__global__ __launch_bounds__(256) void prep_zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// column maxima of |x| (bf16 [M, K]) and |w| (fp32 [N, K]) into amax[0 .. K)
// and amax[K .. 2K); block (bx, by) covers columns 256 bx .. and rows
// rows_per_block by ..
constexpr int kPrepRows = 64;
constexpr int64_t kMaxGridY = 65535;

__global__ __launch_bounds__(256) void prep_colmax_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                          const float* __restrict__ w, int64_t N, int64_t K,
                                                          int64_t rows_per_block, uint32_t* amax) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  uint32_t mx = 0u, mw = 0u;
  for (int64_t r = r0; r < r0 + rows_per_block; ++r) {
    if (r < M) mx = max(mx, (uint32_t)(x[r * K + k] & 0x7fffu) << 16);
    if (r < N) mw = max(mw, __float_as_uint(w[r * K + k]) & 0x7fffffffu);
  }
  if (r0 < M) atomicMax(amax + k, mx);
  if (r0 < N) atomicMax(amax + K + k, mw);
}

__global__ __launch_bounds__(256) void prep_smooth_kernel(const uint32_t* amax, int64_t K, uint16_t* smooth) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const double ax = (double)__uint_as_float(amax[k]);
  const double aw = (double)__uint_as_float(amax[K + k]);
  double lam = __dsqrt_rn(__ddiv_rn(ax, aw));
  if (!(isfinite(lam) && lam > 0.0)) lam = 1.0;
  smooth[k] = bf16_from_f64(lam);
}

// tensor maximum of |r| (fp32, n values, n a multiple of 4, 16-byte
// aligned) into *amax: 16-byte loads, grid-stride, one atomic per workgroup
// (atomics on one address serialize)
__global__ __launch_bounds__(256) void prep_absmax_kernel(const float* __restrict__ r, int64_t n, uint32_t* amax) {
  __shared__ uint32_t wmax[4];
  uint32_t m = 0u;
  const int64_t n4 = n >> 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = *(const u32x4*)(r + 4 * i);
    m = max(m, max(max(v[0] & 0x7fffffffu, v[1] & 0x7fffffffu), max(v[2] & 0x7fffffffu, v[3] & 0x7fffffffu)));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

// One thread per group: G fp32 values of row n -> G/2 code bytes and a scale.
template <int PREC>
__global__ __launch_bounds__(256) void prep_pack_kernel(const float* __restrict__ r, int64_t N, int64_t K,
                                                        uint8_t* __restrict__ packed, void* scales,
                                                        const uint32_t* amax_t, float* wtscale) {
  constexpr int G = PREC == kInt4 ? 64 : 16;
  const int64_t gpr = K / G;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // nvfp4 tensor scale (1 for an all-zero tensor)
  float t = 1.f, six_t = 6.f;
  bool tensor_zero = false;
  if constexpr (PREC == kNvfp4) {
    const float at = __uint_as_float(*amax_t);
    tensor_zero = !(at >= kTiny);
    if (!tensor_zero) {
      t = __fdiv_rn(at, 2688.0f);
      six_t = __fmul_rn(6.0f, t);
    }
  }
  if (gid == 0 && wtscale) *wtscale = t;
  if (gid >= N * gpr) return;
  const float* src = r + gid * G;  // group gid of row gid / gpr, columns G (gid % gpr) ..
  float v[G];
#pragma unroll
  for (int i = 0; i < G; i += 4) {
    const f32x4 q = *(const f32x4*)(src + i);
    v[i] = q[0];
    v[i + 1] = q[1];
    v[i + 2] = q[2];
    v[i + 3] = q[3];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < G; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint8_t* dst = packed + gid * (G / 2);
  if constexpr (PREC == kInt4) {
    const bool zero = !(amax >= kTiny);
    const uint32_t sbits = zero ? 0u : f32_to_bf16_bits(__fdiv_rn(amax, 7.0f));
    const float s = __uint_as_float(sbits << 16);
    const bool z = zero || s == 0.f;
    const float inv = z ? 0.f : __fdiv_rn(1.0f, s);
#pragma unroll
    for (int c = 0; c < G / 8; ++c) {
      uint32_t word = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float tq = __fmul_rn(v[8 * c + j], inv);
        const uint32_t mag = (uint32_t)fminf(__builtin_rintf(fabsf(tq)), 7.0f);
        const uint32_t nib = mag | ((__float_as_uint(tq) >> 28) & 8u);
        word |= nib << (4 * j);
      }
      *(uint32_t*)(dst + 4 * c) = z ? 0u : word;
    }
    ((uint16_t*)scales)[gid] = (uint16_t)(z ? 0u : sbits);
  } else {
    uint32_t s8 = 0u;
    float S = 0.f;
    if (!tensor_zero) {
      const float sf = __fdiv_rn(amax, six_t);
      s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(sf, 448.0f), 0.0f, 0, false) & 0xffu;
      S = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)s8, 0), t);
    }
    const bool z = tensor_zero || !(amax >= kTiny) || S == 0.f;
    const float inv = z ? 0.f : __fdiv_rn(1.0f, S);
    uint32_t cw0 = 0u, cw1 = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t0 = __fmul_rn(v[2 * j], inv);
      const float t1 = __fmul_rn(v[2 * j + 1], inv);
      const uint32_t byte = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t0, t1, 1.0f, 0) & 0xffu;
      if (j < 4) cw0 |= byte << (8 * j);
      else cw1 |= byte << (8 * (j - 4));
    }
    *(u32x2*)dst = z ? u32x2{0u, 0u} : u32x2{cw0, cw1};
    ((uint8_t*)scales)[gid] = (uint8_t)(z ? 0u : s8);
  }
}

static unsigned grid_for(int64_t n, int64_t cap) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > cap ? cap : b));
}

hipError_t launch_smooth_factors(const SmoothArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prep_zero_u32_kernel, dim3(grid_for(2 * a.K, 1024)), dim3(256), 0, s, a.amax, 2 * a.K);
  const int64_t rows = a.M > a.N ? a.M : a.N;
  int64_t rpb = kPrepRows;
  if ((rows + rpb - 1) / rpb > kMaxGridY) rpb = (rows + kMaxGridY - 1) / kMaxGridY;
  const dim3 grid((unsigned)((a.K + 255) / 256), (unsigned)((rows + rpb - 1) / rpb));
  hipLaunchKernelGGL(prep_colmax_kernel, grid, dim3(256), 0, s, (const uint16_t*)a.x, a.M, a.w, a.N, a.K, rpb,
                     a.amax);
  hipLaunchKernelGGL(prep_smooth_kernel, dim3(grid_for(a.K, 1 << 20)), dim3(256), 0, s, (const uint32_t*)a.amax,
                     a.K, (uint16_t*)a.smooth);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const PackArgs& a, hipStream_t s) {
  const int64_t G = a.precision == kInt4 ? 64 : 16;
  const int64_t groups = a.N * (a.K / G);
  if (a.precision == kNvfp4) {
    hipLaunchKernelGGL(prep_zero_u32_kernel, dim3(1), dim3(256), 0, s, a.amax, (int64_t)1);
    hipLaunchKernelGGL(prep_absmax_kernel, dim3(grid_for(a.N * a.K / 4, 1024)), dim3(256), 0, s, a.resid,
                       a.N * a.K, a.amax);
    hipLaunchKernelGGL(prep_pack_kernel<kNvfp4>, dim3(grid_for(groups, 1 << 30)), dim3(256), 0, s, a.resid, a.N,
                       a.K, (uint8_t*)a.packed, a.scales, (const uint32_t*)a.amax, a.wtscale);
  } else {
    hipLaunchKernelGGL(prep_pack_kernel<kInt4>, dim3(grid_for(groups, 1 << 30)), dim3(256), 0, s, a.resid, a.N,
                       a.K, (uint8_t*)a.packed, a.scales, (const uint32_t*)a.amax, a.wtscale);
  }
  return hipGetLastError();
}

}  // namespace svdq
