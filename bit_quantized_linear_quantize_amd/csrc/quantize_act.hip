// Kernel 1 of the SVDQ W4A4 linear: smoothing, per-token group quantization
// of the activations to 4 bits, and the low-rank down projection
// lora_act = X_hat lora_down^T, fused in one pass over X.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table (int4 with
// group 64, nvfp4 with group 16, each with an SVDQ low-rank correction) and
// the news article's description of the low-rank branch as a 16-bit path.
// Numeric readings (the pages name the formats only):
//   X_hat = fl32(x * fl32(1/smooth));
//   int4 : s = bf16(fl32(amax/7)), q = rne(fl32(X_hat * fl32(1/s))), |q| <= 7,
//          sign-magnitude nibble (bit 3 = sign bit of the product);
//   nvfp4: s8 = E4M3(fl32(amax/6)) (round-nearest-even, saturating),
//          code = E2M1(fl32(X_hat * fl32(1/dec(s8)))), tensor scale 1;
//   groups with amax < 2^-100 (or a zero E4M3 scale) get scale 0 and codes 0.
//
// Work layout (gfx950, wave64): a workgroup of W waves owns 16 token rows and
// all K (W = 16 for ranks up to 32, else 8); wave w handles the 64-column
// chunks w, w+W, w+2W, ...  Inside a wave,
// lane (r = lane%16, q = lane/16) holds 16 consecutive columns 64c+16q..+15 of
// row r.  That is exactly one nvfp4 group per lane, a quarter of an int4 group
// (amax then needs two cross-lane max steps), and the A-operand slot group q
// of the 16x16x32 bf16 matrix instruction used for the low-rank product.  X_hat
// is split into bf16 hi + lo parts so the low-rank product keeps ~16 bits.
// The per-wave low-rank partials are summed in LDS in a fixed order
// (deterministic).  Loads of X are 16 bytes per lane, several chunks in
// flight; the first ones are issued before the workgroup computes its table
// of 1 / smooth.
//
// Outputs.  The parity export writes packed nibbles (low nibble = even
// column), the group scales and lora_act.  Inside svdq_w4a4_linear the kernel
// instead writes the operand the product kernel reads: int4 the codes q as
// fp8 E4M3 bytes (exact: |q| <= 7) and the group scales as fp32, nvfp4 the
// activations dequantized to e2m1 * dec(s8) in fp16 (always exact).

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int kK1Rows = 16;

// Waves per workgroup (they split K) and 64-column chunks in flight per wave.
// Ranks up to 32 run 16 waves (4 per SIMD, within 128 VGPRs) with two chunks
// in flight; larger ranks need more registers for the low-rank operands and
// run 8 waves.
template <int RB>
struct K1Shape {
  static constexpr int waves = RB <= 2 ? 16 : 8;
  static constexpr int prefetch = 2;
};

// K slices (the linear, few rows): workgroup b takes row block b / S and the
// chunks [c0, c0 + C) of K slice b % S (C = K/64 / S), with one wave per
// chunk up to the usual count; its low-rank sums are one fp32 partial
// lora_part[slice, M, rank] (the slices are added in order afterwards).
// With S = 1 it is the kernel above.  The wave count is the launch's.
template <int PREC, int RB, bool LINEAR>
__global__ __launch_bounds__(64 * K1Shape<RB>::waves) void quantize_act_lora_down_kernel(QuantActArgs args) {
  const int kK1Waves = (int)(blockDim.x >> 6);
  const int kK1Threads = (int)blockDim.x;
  extern __shared__ float lds[];
  constexpr int PF = K1Shape<RB>::prefetch;
  constexpr int NB = RB > 0 ? RB : 1;
  const int M = (int)args.M, K = (int)args.K;
  const uint16_t* __restrict__ x = (const uint16_t*)args.x;
  const uint16_t* __restrict__ smooth = (const uint16_t*)args.smooth;
  const uint16_t* __restrict__ lora_down = (const uint16_t*)args.lora_down;
  uint8_t* __restrict__ codes = (uint8_t*)args.codes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int r = lane & 15;
  const int q = lane >> 4;
  const int S = LINEAR ? args.k_slices : 1;
  const int slice = (int)blockIdx.x % S;
  const int row = ((int)blockIdx.x / S) * kK1Rows + r;
  const bool row_ok = row < M;
  const uint16_t* xr = x + (size_t)(row_ok ? row : M - 1) * K;
  const int nchunks = (K >> 6) / S;   // chunks of this slice
  const int c0 = slice * nchunks;     // its first chunk
  const int kb = c0 * 64;             // its first column

  // X_hat of the lane's 16 columns k0 .. k0+15
  auto smooth16 = [&](const u32x4* xb, int k0, float* xh) {
    const f32x4* mu4 = (const f32x4*)(lds + (k0 - kb));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = xb[h][i];
        const f32x4 mu = mu4[h * 2 + (i >> 1)];
        xh[h * 8 + 2 * i] = __fmul_rn(bf16_lo(w), mu[(2 * i) & 3]);
        xh[h * 8 + 2 * i + 1] = __fmul_rn(bf16_hi(w), mu[(2 * i + 1) & 3]);
      }
    }
  };
  // int4: the group (the four lanes q = 0..3 of the row) scale, returned as
  // bf16 bits (0 for a zero group), and 1/s (0 for a zero group)
  auto int4_scale = [&](const float* xh, float& inv) -> uint32_t {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
    amax = wave_max_xor(amax, 16);
    amax = wave_max_xor(amax, 32);
    const bool zero = !(amax >= kTiny);
    const uint32_t sbits = zero ? 0u : f32_to_bf16_bits(__fdiv_rn(amax, 7.0f));
    inv = zero ? 0.f : __fdiv_rn(1.0f, __uint_as_float(sbits << 16));
    return sbits;
  };
  // int4: the lane's 16 sign-magnitude codes of q = rne(x / s)
  auto int4_codes = [&](const float* xh, float inv, uint32_t sbits, uint32_t& cw0, uint32_t& cw1) {
    cw0 = 0;
    cw1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = __fmul_rn(xh[i], inv);
      // |t| < 7.5, so adding 1.5 * 2^23 rounds it to the nearest integer
      // (ties to even) in the low mantissa bits
      const uint32_t m = __float_as_uint(__fadd_rn(fabsf(t), 12582912.0f));
      const uint32_t nib = (m & 7u) | ((__float_as_uint(t) >> 28) & 8u);
      if (i < 8) cw0 |= nib << (4 * i);
      else cw1 |= nib << (4 * (i - 8));
    }
    cw0 = sbits == 0u ? 0u : cw0;
    cw1 = sbits == 0u ? 0u : cw1;
  };
  // int4, product operand: the 16 codes q = rne(x / s) of the lane as fp8
  // E4M3 bytes (every integer |q| <= 7 is exact; a negative value that rounds
  // to 0 gives -0, as the sign-magnitude code does)
  auto int4_q8 = [&](const float* xh, float inv) -> u32x4 {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float q0 = __builtin_rintf(__fmul_rn(xh[4 * p], inv)), q1 = __builtin_rintf(__fmul_rn(xh[4 * p + 1], inv));
      const float q2 = __builtin_rintf(__fmul_rn(xh[4 * p + 2], inv)), q3 = __builtin_rintf(__fmul_rn(xh[4 * p + 3], inv));
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      r[p] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
    }
    return r;
  };

  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xbuf[PF][2];
  u32x4 lbuf[PF][NB][2];

  auto issue = [&](int slot, int c) {
    if (c < nchunks) {
      const int k0 = (c0 + c) * 64 + q * 16;
      xbuf[slot][0] = *(const u32x4*)(xr + k0);
      xbuf[slot][1] = *(const u32x4*)(xr + k0 + 8);
      if constexpr (RB > 0) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint16_t* lr = lora_down + (size_t)(b * 16 + r) * K + k0;
          lbuf[slot][b][0] = *(const u32x4*)(lr);
          lbuf[slot][b][1] = *(const u32x4*)(lr + 8);
        }
      }
    }
  };

#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p, wave + p * kK1Waves);

  // 1 / smooth for every input channel of the slice (IEEE division, one per
  // channel), computed while the first chunks are in flight
  for (int k = tid; k < nchunks * 64; k += kK1Threads) lds[k] = __fdiv_rn(1.0f, bf16_bits_to_f32(smooth[kb + k]));
  __syncthreads();

  for (int base = wave; base < nchunks; base += PF * kK1Waves) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int cl = base + p * kK1Waves;  // chunk of the slice
      const int c = c0 + cl;               // chunk of K
      if (cl < nchunks) {
        const int k0 = c * 64 + q * 16;
        float xh[16];
        smooth16(xbuf[p], k0, xh);

        // ---- quantize -----------------------------------------------------
        uint32_t cw0 = 0, cw1 = 0;
        if constexpr (PREC == kInt4) {
          float inv;
          const uint32_t sbits = int4_scale(xh, inv);
          const float sv = __uint_as_float(sbits << 16);
          if constexpr (LINEAR) {
            if (row_ok) {
              // (a zero group gets codes 0, as in the packed export)
              const u32x4 z = {0u, 0u, 0u, 0u};
              *(u32x4*)((uint8_t*)args.act_op + (size_t)row * K + k0) = sbits == 0u ? z : int4_q8(xh, inv);
              if (q == 0) {
                if (args.scale_bf16) ((uint16_t*)args.act_scale)[(size_t)row * (K >> 6) + c] = (uint16_t)sbits;
                else args.act_scale[(size_t)row * (K >> 6) + c] = sv;
              }
            }
          } else {
            int4_codes(xh, inv, sbits, cw0, cw1);
            if (row_ok && q == 0) ((uint16_t*)args.scales)[(size_t)row * (K >> 6) + c] = (uint16_t)sbits;
          }
        } else {
          float S;
          const uint32_t s8 = nvfp4_quant16(xh, cw0, cw1, S);
          if constexpr (LINEAR) {
            // the product operand e2m1 * dec(s8): an exact fp16 (|v| <= 2688, >= 2^-10)
            if (row_ok) {
              const _Float16 S16 = (_Float16)S;
              _Float16* dst = (_Float16*)args.act_op + (size_t)row * K + k0;
              *(f16x8*)dst = e2m1x8_to_f16_scaled(cw0, S16);
              *(f16x8*)(dst + 8) = e2m1x8_to_f16_scaled(cw1, S16);
            }
          } else if (row_ok) {
            ((uint8_t*)args.scales)[(size_t)row * (K >> 4) + 4 * c + q] = (uint8_t)s8;
          }
        }
        if (row_ok && !LINEAR) *(u32x2*)(codes + (size_t)row * (K >> 1) + (k0 >> 1)) = u32x2{cw0, cw1};

        // ---- low-rank down projection (bf16 hi + lo, fp32 accumulate) ------
        if constexpr (RB > 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            // hi = bf16(v), lo = bf16(v - hi), both round to nearest even,
            // converted two at a time
            u32x4 hi4, lo4;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const float a = xh[8 * j + 2 * p], b = xh[8 * j + 2 * p + 1];
              const uint32_t h = bf16x2_rne(a, b);
              hi4[p] = h;
              lo4[p] = bf16x2_rne(__fsub_rn(a, bf16_lo(h)), __fsub_rn(b, bf16_hi(h)));
            }
            const bf16x8 ahi = __builtin_bit_cast(bf16x8, hi4);
            const bf16x8 alo = __builtin_bit_cast(bf16x8, lo4);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
              const bf16x8 bop = __builtin_bit_cast(bf16x8, lbuf[p][b][j]);
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bop, acc[b], 0, 0, 0);
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bop, acc[b], 0, 0, 0);
            }
          }
        }
        issue(p, cl + PF * kK1Waves);
      }
    }
  }

  // ---- reduce the low-rank partials of the waves (fixed order) -------------
  if constexpr (RB > 0) {
    constexpr int rank = RB * 16;
    __syncthreads();  // everyone is done with the 1/smooth table
    float* red = lds;  // [wave][16 rows][rank]
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[(wave * kK1Rows + q * 4 + j) * rank + b * 16 + r] = acc[b][j];
    __syncthreads();
    // (one slice: lora_act itself; else this slice's partial)
    float* out = S > 1 ? args.lora_part + (size_t)slice * M * rank : args.lora_act;
    for (int o = tid; o < kK1Rows * rank; o += kK1Threads) {
      const int rr = o / rank;
      const int cc = o - rr * rank;
      float s = 0.f;
      for (int w = 0; w < kK1Waves; ++w) s += red[(w * kK1Rows + rr) * rank + cc];
      const int grow = ((int)blockIdx.x / S) * kK1Rows + rr;
      if (grow < M) out[(size_t)grow * rank + cc] = s;
    }
  }
}

template <int PREC, int RB, bool LINEAR>
static hipError_t launch_k1(const QuantActArgs& a, hipStream_t stream) {
  const int rank = RB * 16;
  const int S = LINEAR ? a.k_slices : 1;
  const int chunks = (int)(a.K >> 6) / S;  // per slice
  const int waves = chunks < K1Shape<RB>::waves ? chunks : K1Shape<RB>::waves;
  size_t lds = (size_t)chunks * 64 * sizeof(float);
  const size_t red = (size_t)waves * kK1Rows * rank * sizeof(float);
  if (red > lds) lds = red;
  const unsigned blocks = (unsigned)((a.M + kK1Rows - 1) / kK1Rows) * (unsigned)S;
  hipLaunchKernelGGL((quantize_act_lora_down_kernel<PREC, RB, LINEAR>), dim3(blocks), dim3(64 * waves), lds,
                     stream, a);
  return hipGetLastError();
}

template <int PREC, bool LINEAR>
static hipError_t dispatch_rank(const QuantActArgs& a, hipStream_t s) {
  switch (a.rank / 16) {
    case 0: return launch_k1<PREC, 0, LINEAR>(a, s);
    case 1: return launch_k1<PREC, 1, LINEAR>(a, s);
    case 2: return launch_k1<PREC, 2, LINEAR>(a, s);
    case 3: return launch_k1<PREC, 3, LINEAR>(a, s);
    case 4: return launch_k1<PREC, 4, LINEAR>(a, s);
    case 5: return launch_k1<PREC, 5, LINEAR>(a, s);
    case 6: return launch_k1<PREC, 6, LINEAR>(a, s);
    case 7: return launch_k1<PREC, 7, LINEAR>(a, s);
    case 8: return launch_k1<PREC, 8, LINEAR>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_act(const QuantActArgs& a, hipStream_t stream) {
  const bool linear = a.act_op != nullptr;
  if (a.k_slices < 1 || (a.K >> 6) % a.k_slices || (a.k_slices > 1 && (!linear || (a.rank > 0 && !a.lora_part))))
    return hipErrorInvalidValue;
  if (a.precision == kInt4)
    return linear ? dispatch_rank<kInt4, true>(a, stream) : dispatch_rank<kInt4, false>(a, stream);
  return linear ? dispatch_rank<kNvfp4, true>(a, stream) : dispatch_rank<kNvfp4, false>(a, stream);
}

}  // namespace svdq
