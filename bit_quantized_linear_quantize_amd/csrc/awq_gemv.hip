// AWQ W4A16 linear for the small-M adaptive-norm layers.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table, row
// awq_w4a16 (int4 weight-only, group 64); the news article assigns this path to
// the precision-sensitive adaptive-normalization layers.  Reading of the
// format: unsigned codes q (0..15), per-group bf16 scale s and integer
// zero-point z, W = (q - z) s;  Y = X W^T + bias with fp32 accumulation.
//
// gfx950 design -- bandwidth-bound: 4.5 bits per weight streamed once per 32
// rows of X.
// * A workgroup owns 32 weight rows (output columns); its 4 waves split K in
//   four contiguous ranges, so 4 x N/32 waves stream independently.  Each lane
//   issues all of its 16-byte code loads (one per group in its range) before
//   computing, so the whole weight matrix is in flight at once.
// * Lane (n = lane%32, h = lane/32) covers columns 64g + 32h .. +31 of weight
//   row n: four 32x32x16 bf16 matrix instructions per group, each mixing only
//   columns of that group.
// * Codes become bf16 operands 128 + q (0x4300 | q is the bit pattern of
//   128 + q) with one v_perm and one OR per pair.  A second operand set holds
//   -(128 + z) in every slot, so the same accumulator collects
//   sum_k x (128 + q) - sum_k x (128 + z) = sum_k x (q - z) exactly in the
//   matrix unit (exact bf16 products, fp32 sums), and the scale needs one FMA
//   per output: acc += t * s.
// * Rows of X beyond M are zero; the epilogue skips blocks of rows beyond M.
//   The four K-range partials are summed in LDS in a fixed order.

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int kAwqWaves = 4;     // K ranges per workgroup
constexpr int kAwqMaxG = 16;     // groups per wave held in registers at once

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
  __shared__ float part[kAwqWaves][32][33];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = (int)args.M, K = (int)args.K, N = (int)args.N;
  const int G = K >> 6;
  const int K2 = K >> 1;
  const int m0 = blockIdx.y * 32;
  const int rows = min(32, M - m0);
  const uint16_t* __restrict__ x = (const uint16_t*)args.x;

  const int n_l = lane & 31;
  const int h = lane >> 5;
  const int n = blockIdx.x * 32 + n_l;
  const int nc = min(n, N - 1);
  // this wave's contiguous range of groups
  const int gpw = (G + kAwqWaves - 1) / kAwqWaves;
  const int g0 = min(G, wave * gpw);
  const int g1 = min(G, g0 + gpw);
  const uint8_t* wrow = (const uint8_t*)args.w_codes + (size_t)nc * K2 + h * 16;
  const uint16_t* srow = (const uint16_t*)args.scales + (size_t)nc * G;
  const uint16_t* zrow = (const uint16_t*)args.zeros + (size_t)nc * G;
  const bool x_ok = n_l < rows;
  const uint16_t* xrow = x + (size_t)(m0 + (x_ok ? n_l : 0)) * K + h * 32;

  f32x16 acc = {};
  const f32x16 zero16 = {};
  for (int gb = g0; gb < g1; gb += kAwqMaxG) {
    // every load of this batch is issued before any use, so only one memory
    // latency is exposed per batch (codes, scales and zero-points)
    u32x4 wbuf[kAwqMaxG];
    uint16_t sbuf[kAwqMaxG], zbuf[kAwqMaxG];
#pragma unroll
    for (int p = 0; p < kAwqMaxG; ++p)
      if (gb + p < g1) wbuf[p] = *(const u32x4*)(wrow + (gb + p) * 32);
#pragma unroll
    for (int p = 0; p < kAwqMaxG; ++p)
      if (gb + p < g1) {
        sbuf[p] = srow[gb + p];
        zbuf[p] = zrow[gb + p];
      }
    // rows of X for the A operand: 64 bytes per lane and group, two groups ahead
    u32x4 xbuf[3][4];
    auto load_x = [&](int slot, int g) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xbuf[slot][j] = (x_ok && g < g1) ? *(const u32x4*)(xrow + g * 64 + j * 8) : u32x4{0u, 0u, 0u, 0u};
    };
    load_x(0, gb);
    load_x(1, gb + 1);
#pragma unroll
    for (int p = 0; p < kAwqMaxG; ++p) {
      const int g = gb + p;
      if (g >= g1) continue;
      if (p + 2 < kAwqMaxG) load_x((p + 2) % 3, g + 2);
      const float s = bf16_bits_to_f32(sbuf[p]);
      const uint32_t zb = f32_to_bf16_bits(-(128.0f + bf16_bits_to_f32(zbuf[p])));  // exact
      const uint32_t zz = zb | (zb << 16);
      const bf16x8 zop = __builtin_bit_cast(bf16x8, u32x4{zz, zz, zz, zz});
      f32x16 t = zero16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, xbuf[p % 3][j]);
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, awq_operand(wbuf[p][j]), t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, zop, t, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e >> 2) * 8 < rows) acc[e] = __builtin_fmaf(t[e], s, acc[e]);  // wave-uniform skip
    }
  }

  // ---- sum the K-range partials in a fixed order, add bias, store -----------
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = (e >> 2) * 8 + h * 4 + (e & 3);
    part[wave][m][n_l] = acc[e];
  }
  __syncthreads();
  const uint16_t* bias = (const uint16_t*)args.bias;
  uint16_t* out = (uint16_t*)args.out;
  for (int o = tid; o < 32 * 32; o += 256) {
    const int m = o >> 5, c = o & 31;
    const int col = blockIdx.x * 32 + c;
    if (m < rows && col < N) {
      float v = part[0][m][c];
#pragma unroll
      for (int w = 1; w < kAwqWaves; ++w) v += part[w][m][c];
      if (bias) v += bf16_bits_to_f32(bias[col]);
      out[(size_t)(m0 + m) * N + col] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

hipError_t launch_awq_gemv(const AwqArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.N + 31) / 32), (unsigned)((a.M + 31) / 32));
  hipLaunchKernelGGL(awq_w4a16_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace svdq
