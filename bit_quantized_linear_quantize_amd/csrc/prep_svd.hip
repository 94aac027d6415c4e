// Offline weight preparation, the low-rank split on the GPU: the products of
// a randomized range finder with subspace iteration (Halko, Martinsson and
// Tropp, "Finding structure with randomness", 2011: Algorithms 4.3 and 4.4)
// over the smoothed weight W_hat = W * smooth, and the residual
// R = W_hat - lora_up lora_down that the packer quantizes.  The host side
// (api.cpp) does the l x l factorizations (l = rank + oversampling) in fp64.
//
// Everything is fp64 with separate multiplies and adds in a fixed order (no
// fused multiply-add: the build disables contraction), so a preparation is
// reproducible bit for bit, and the residual equals the CPU reference's for
// the same bf16 factors:
//   W_hat[n, k] = fl64(w[n, k] * smooth[k])              (exact: 24 x 8 bits)
//   L[n, k]     = sum_{j = 0 .. r-1} fl64(up[n, j] * down[j, k]), in order j
//   R[n, k]     = fl32(fl64(W_hat[n, k] - L[n, k]))
// The matrices of the range finder are dense row-major fp64; W_hat is never
// stored, each product forms it from the fp32 weight and the bf16 factors.

#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

namespace {

constexpr int kThreadsP = 256;
constexpr int kMaxL = kPrepMaxL;

// A(n, c) of the products: the smoothed weight (R = N rows, C = K columns)
// or a dense fp64 matrix with leading dimension ld.
struct SrcW {
  const float* w;
  const uint16_t* smooth;
  int64_t K;
  __device__ __forceinline__ double operator()(int64_t n, int64_t c) const {
    return __dmul_rn((double)w[n * K + c], (double)bf16_bits_to_f32(smooth[c]));
  }
};
struct SrcD {
  const double* p;
  int64_t ld;
  __device__ __forceinline__ double operator()(int64_t n, int64_t c) const { return p[n * ld + c]; }
};

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014) as a counter-based generator: output i of stream `seed`.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Omega[k, j] (K x l) standard normal by the Box-Muller transform of two
// uniform draws in (0, 1] (53 bits each).
__global__ __launch_bounds__(kThreadsP) void prep_gauss_kernel(double* omega, int64_t n, uint64_t seed) {
  const int64_t i = (int64_t)blockIdx.x * kThreadsP + threadIdx.x;
  if (i >= n) return;
  const double u1 = (double)((splitmix64(seed, 2 * i) >> 11) + 1) * 0x1p-53;
  const double u2 = (double)(splitmix64(seed, 2 * i + 1) >> 11) * 0x1p-53;
  omega[i] = sqrt(-2.0 * log(u1)) * cospi(2.0 * u2);
}

// out[n, j] = sum_c A(n, c) B[c, j] (n < R, j < l; B dense [C, l]).  A
// workgroup owns 16 rows and all l columns; C is walked in chunks of 64 with
// the A tile and the B chunk in LDS; the sum is taken in order of c.
template <class Src>
__global__ __launch_bounds__(kThreadsP) void prep_ab_kernel(Src A, int64_t R, int64_t C, const double* __restrict__ B,
                                                           int l, double* __restrict__ out) {
  __shared__ double a_t[16][65];
  __shared__ double b_t[64 * kMaxL];
  const int t = threadIdx.x;
  const int r = t >> 4, jj = t & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  double acc[kMaxL / 16];
#pragma unroll
  for (int i = 0; i < kMaxL / 16; ++i) acc[i] = 0.0;
  for (int64_t c0 = 0; c0 < C; c0 += 64) {
    const int cw = (int)min<int64_t>(64, C - c0);
    for (int e = t; e < 16 * 64; e += kThreadsP) {
      const int rr = e >> 6, cc = e & 63;
      a_t[rr][cc] = (n0 + rr < R && cc < cw) ? A(n0 + rr, c0 + cc) : 0.0;
    }
    for (int e = t; e < cw * l; e += kThreadsP) b_t[e] = B[c0 * l + e];
    __syncthreads();
    for (int c = 0; c < cw; ++c) {
      const double av = a_t[r][c];
#pragma unroll
      for (int i = 0; i < kMaxL / 16; ++i) {
        const int j = jj + 16 * i;
        if (j < l) acc[i] = __dadd_rn(acc[i], __dmul_rn(av, b_t[c * l + j]));
      }
    }
    __syncthreads();
  }
  if (n0 + r < R) {
#pragma unroll
    for (int i = 0; i < kMaxL / 16; ++i) {
      const int j = jj + 16 * i;
      if (j < l) out[(n0 + r) * l + j] = acc[i];
    }
  }
}

// part[s, c, j] = sum over rows n of slice s of A(n, c) B[n, j] (c < C, j < l;
// B dense [R, l]); slice s is rows [s rows_per, (s + 1) rows_per).  A
// workgroup owns 64 columns c of one slice; thread t takes column t % 64 and
// the columns j = t / 64 + 4 i.  Rows are walked in order, 32 at a time with
// the B rows in LDS.
template <class Src>
__global__ __launch_bounds__(kThreadsP) void prep_atb_kernel(Src A, int64_t R, int64_t C, const double* __restrict__ B,
                                                            int l, int64_t rows_per, double* __restrict__ part) {
  __shared__ double b_t[32 * kMaxL];
  const int t = threadIdx.x;
  const int cc = t & 63, jg = t >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + cc;
  const int64_t s = blockIdx.y;
  const int64_t r0 = s * rows_per, r1 = min(R, r0 + rows_per);
  double acc[kMaxL / 4];
#pragma unroll
  for (int i = 0; i < kMaxL / 4; ++i) acc[i] = 0.0;
  for (int64_t n0 = r0; n0 < r1; n0 += 32) {
    const int rows = (int)min<int64_t>(32, r1 - n0);
    for (int e = t; e < rows * l; e += kThreadsP) b_t[e] = B[n0 * l + e];
    __syncthreads();
    if (c < C) {
      for (int rr = 0; rr < rows; ++rr) {
        const double av = A(n0 + rr, c);
#pragma unroll
        for (int i = 0; i < kMaxL / 4; ++i) {
          const int j = jg + 4 * i;
          if (j < l) acc[i] = __dadd_rn(acc[i], __dmul_rn(av, b_t[rr * l + j]));
        }
      }
    }
    __syncthreads();
  }
  if (c < C) {
#pragma unroll
    for (int i = 0; i < kMaxL / 4; ++i) {
      const int j = jg + 4 * i;
      if (j < l) part[(s * C + c) * l + j] = acc[i];
    }
  }
}

// out[i] = sum_s part[s, i] in order of s
__global__ __launch_bounds__(kThreadsP) void prep_sum_slices_kernel(const double* __restrict__ part, int64_t n,
                                                                    int slices, double* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreadsP + threadIdx.x;
  if (i >= n) return;
  double a = 0.0;
  for (int s = 0; s < slices; ++s) a = __dadd_rn(a, part[s * n + i]);
  out[i] = a;
}

// dst (bf16 bits) = src (fp64 [rows, cols], leading dimension ld), optionally
// transposed: dst[c, r] when transpose, else dst[r, c]
__global__ __launch_bounds__(kThreadsP) void prep_to_bf16_kernel(const double* __restrict__ src, int64_t rows,
                                                                 int64_t cols, int64_t ld, bool transpose,
                                                                 uint16_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * kThreadsP + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, c = i - r * cols;
  const uint16_t b = bf16_from_f64(src[r * ld + c]);
  if (transpose) dst[c * rows + r] = b;
  else dst[r * cols + c] = b;
}

// R[n, k] = fl32(W_hat[n, k] - sum_j up[n, j] down[j, k]) (the sum in order
// of j, separate multiplies and adds); up bf16 [N, r], down bf16 [r, K]
__global__ __launch_bounds__(kThreadsP) void prep_residual_kernel(const float* __restrict__ w,
                                                                  const uint16_t* __restrict__ smooth,
                                                                  const uint16_t* __restrict__ up,
                                                                  const uint16_t* __restrict__ down, int64_t N,
                                                                  int64_t K, int rank, float* __restrict__ resid) {
  for (int64_t i = (int64_t)blockIdx.x * kThreadsP + threadIdx.x; i < N * K; i += (int64_t)gridDim.x * kThreadsP) {
    const int64_t n = i / K, k = i - n * K;
    double low = 0.0;
    for (int j = 0; j < rank; ++j)
      low = __dadd_rn(low, __dmul_rn((double)bf16_bits_to_f32(up[n * rank + j]),
                                     (double)bf16_bits_to_f32(down[(int64_t)j * K + k])));
    const double wh = __dmul_rn((double)w[i], (double)bf16_bits_to_f32(smooth[k]));
    resid[i] = (float)__dsub_rn(wh, low);
  }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreadsP - 1) / kThreadsP); }

}  // namespace

hipError_t launch_prep_gauss(double* omega, int64_t n, uint64_t seed, hipStream_t s) {
  hipLaunchKernelGGL(prep_gauss_kernel, dim3(blocks_for(n)), dim3(kThreadsP), 0, s, omega, n, seed);
  return hipGetLastError();
}

// out [R, l] = A [R, C] B [C, l]; A the smoothed weight (w, smooth given) or
// the dense fp64 a [R, C]
hipError_t launch_prep_ab(const PrepSrc& a, int64_t R, int64_t C, const double* B, int l, double* out,
                          hipStream_t s) {
  if (l < 1 || l > kMaxL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((R + 15) / 16));
  if (a.w) {
    hipLaunchKernelGGL((prep_ab_kernel<SrcW>), grid, dim3(kThreadsP), 0, s, SrcW{a.w, (const uint16_t*)a.smooth, C}, R, C, B, l,
                       out);
  } else {
    hipLaunchKernelGGL((prep_ab_kernel<SrcD>), grid, dim3(kThreadsP), 0, s, SrcD{a.dense, C}, R, C, B, l, out);
  }
  return hipGetLastError();
}

// out [C, l] = A^T B for A [R, C] (as above) and B [R, l]: `slices` row
// slices into part [slices, C, l], then summed in order of slice into out
hipError_t launch_prep_atb(const PrepSrc& a, int64_t R, int64_t C, const double* B, int l, int slices, double* part,
                           double* out, hipStream_t s) {
  if (l < 1 || l > kMaxL || slices < 1) return hipErrorInvalidValue;
  const int64_t rows_per = (R + slices - 1) / slices;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)slices);
  if (a.w) {
    hipLaunchKernelGGL((prep_atb_kernel<SrcW>), grid, dim3(kThreadsP), 0, s, SrcW{a.w, (const uint16_t*)a.smooth, C}, R, C, B, l,
                       rows_per, part);
  } else {
    hipLaunchKernelGGL((prep_atb_kernel<SrcD>), grid, dim3(kThreadsP), 0, s, SrcD{a.dense, C}, R, C, B, l,
                       rows_per, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = C * l;
  hipLaunchKernelGGL(prep_sum_slices_kernel, dim3(blocks_for(n)), dim3(kThreadsP), 0, s, part, n, slices, out);
  return hipGetLastError();
}

hipError_t launch_prep_to_bf16(const double* src, int64_t rows, int64_t cols, int64_t ld, bool transpose,
                               uint16_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(prep_to_bf16_kernel, dim3(blocks_for(rows * cols)), dim3(kThreadsP), 0, s, src, rows, cols, ld,
                     transpose, dst);
  return hipGetLastError();
}

hipError_t launch_prep_residual(const float* w, const void* smooth, const void* up, const void* down, int64_t N,
                                int64_t K, int rank, float* resid, hipStream_t s) {
  const dim3 grid((unsigned)std::min<int64_t>(blocks_for(N * K), 65536));
  hipLaunchKernelGGL(prep_residual_kernel, grid, dim3(kThreadsP), 0, s, w, (const uint16_t*)smooth,
                     (const uint16_t*)up, (const uint16_t*)down, N, K, rank, resid);
  return hipGetLastError();
}

}  // namespace svdq
