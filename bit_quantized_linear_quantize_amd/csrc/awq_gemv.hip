// AWQ W4A16 linear for the small-M adaptive-norm layers.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table, row
// awq_w4a16 (int4 weight-only, group 64); the news article assigns this path to
// the precision-sensitive adaptive-normalization layers.  Reading of the
// format: unsigned codes q (0..15), per-group bf16 scale s and integer
// zero-point z, W = (q - z) s;  Y = X W^T + bias with fp32 accumulation.
//
// gfx950 design: bandwidth-bound (4.5 bits per weight streamed once per call).
// One wave owns 32 weight rows (output columns) and all of K; a workgroup has
// 4 waves.  Lane (n = lane%32, h = lane/32) streams 16 bytes of row n per group
// (columns 64g + 32h .. +31), several groups in flight.  Codes become bf16
// operands 128 + q with one v_perm + one OR per pair (0x4300 | q is the bf16
// bit pattern of 128 + q), and one 32x32x16 bf16 matrix instruction per 16
// columns contracts them with up to 32 rows of X.  Per group,
//   sum_k x (q - z) s = s * (P - (128 + z) * sum_k x),
// with P the matrix-instruction result (exact products, fp32 sums) and
// sum_k x precomputed per workgroup in LDS.  Rows of X beyond M are zero and
// skip the epilogue.  X is re-read from L2 by every wave (it is small).

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int kAwqWaves = 4;
constexpr int kAwqPF = 4;  // groups in flight per lane

__device__ __forceinline__ bf16x8 awq_operand(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // nibbles 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // nibbles 1, 3, 5, 7
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;  // (n0, n1)
  r[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;  // (n2, n3)
  r[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u;  // (n4, n5)
  r[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u;  // (n6, n7)
  return __builtin_bit_cast(bf16x8, r);
}

__global__ __launch_bounds__(256) void awq_w4a16_kernel(AwqArgs args) {
  extern __shared__ float xsum[];  // [32 rows][G]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = (int)args.M, K = (int)args.K, N = (int)args.N;
  const int G = K >> 6;
  const int K2 = K >> 1;
  const int m0 = blockIdx.y * 32;
  const int rows = min(32, M - m0);
  const uint16_t* __restrict__ x = (const uint16_t*)args.x;

  // sum of X over each group, for the 128 + q offset of the operands
  for (int o = tid; o < 32 * G; o += 256) {
    const int m = o / G, g = o - m * G;
    float s = 0.f;
    if (m < rows) {
      const u32x4* p = (const u32x4*)(x + (size_t)(m0 + m) * K + g * 64);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const u32x4 w = p[v];
#pragma unroll
        for (int i = 0; i < 4; ++i) s += bf16_lo(w[i]) + bf16_hi(w[i]);
      }
    }
    xsum[o] = s;
  }
  __syncthreads();

  const int n_l = lane & 31;
  const int h = lane >> 5;
  const int n = blockIdx.x * (32 * kAwqWaves) + wave * 32 + n_l;
  const int nc = min(n, N - 1);
  const uint8_t* wrow = (const uint8_t*)args.w_codes + (size_t)nc * K2 + h * 16;
  const uint16_t* srow = (const uint16_t*)args.scales + (size_t)nc * G;
  const uint16_t* zrow = (const uint16_t*)args.zeros + (size_t)nc * G;
  const int xm = m0 + n_l;  // row of X this lane feeds into the A operand
  const bool x_ok = n_l < rows;
  const uint16_t* xrow = x + (size_t)(x_ok ? xm : 0) * K + h * 32;

  f32x16 acc = {};
  const f32x16 zero16 = {};
  u32x4 wbuf[kAwqPF];
#pragma unroll
  for (int p = 0; p < kAwqPF; ++p)
    if (p < G) wbuf[p] = *(const u32x4*)(wrow + p * 32);

  for (int gb = 0; gb < G; gb += kAwqPF) {
#pragma unroll
    for (int p = 0; p < kAwqPF; ++p) {
      const int g = gb + p;
      if (g >= G) break;
      const u32x4 wv = wbuf[p];
      if (g + kAwqPF < G) wbuf[p] = *(const u32x4*)(wrow + (g + kAwqPF) * 32);
      f32x16 P = zero16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 a = {};
        if (x_ok) a = __builtin_bit_cast(bf16x8, *(const u32x4*)(xrow + g * 64 + j * 8));
        P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, awq_operand(wv[j]), P, 0, 0, 0);
      }
      const float s = bf16_bits_to_f32(srow[g]);
      const float zoff = -(128.0f + bf16_bits_to_f32(zrow[g]));
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = (e >> 2) * 8 + h * 4 + (e & 3);
        if ((e >> 2) * 8 < rows) {  // wave-uniform skip of blocks of rows beyond M
          const float t = __builtin_fmaf(zoff, xsum[m * G + g], P[e]);
          acc[e] = __builtin_fmaf(t, s, acc[e]);
        }
      }
    }
  }

  const uint16_t* bias = (const uint16_t*)args.bias;
  const float bv = bias ? bf16_bits_to_f32(bias[nc]) : 0.f;
  uint16_t* out = (uint16_t*)args.out;
  if (n < N) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = (e >> 2) * 8 + h * 4 + (e & 3);
      if (m < rows) out[(size_t)(m0 + m) * N + n] = (uint16_t)f32_to_bf16_bits(acc[e] + bv);
    }
  }
}

hipError_t launch_awq_gemv(const AwqArgs& a, hipStream_t stream) {
  const int G = (int)(a.K >> 6);
  const size_t lds = (size_t)32 * G * sizeof(float);
  dim3 grid((unsigned)((a.N + 32 * kAwqWaves - 1) / (32 * kAwqWaves)), (unsigned)((a.M + 31) / 32));
  hipLaunchKernelGGL(awq_w4a16_kernel, grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace svdq
