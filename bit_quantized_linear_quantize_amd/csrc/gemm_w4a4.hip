// Kernel 2 of the SVDQ W4A4 linear: the 4-bit x 4-bit product with per-group
// scales, plus the low-rank up projection, the bias and the bf16 store.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table (svdq_w4a4:
// int4 with group 64 or nvfp4 with group 16, each with an SVDQ low-rank
// correction); bf16 compute dtype from the "NunchakuLiteQuantizationConfig"
// section.  Y = sum_g P_g * s_x * s_w * wtscale + lora_act lora_up^T + bias.
//
// gfx950 design (wave64, 256 threads = 4 waves, a 128x128 output tile per
// workgroup, 64x64 = 2x2 blocks of 32x32 per wave, 64 columns of K per stage,
// LDS double-buffered with one barrier per stage):
//
// int4  The group (64 k) is exactly one v_mfma_scale_f32_32x32x64_f8f6f4 with
//       fp8 E4M3 operands and unit block scales: the integer codes -7..7 are
//       exact in E4M3, so the fp32 result is the exact integer partial P_g.
//       Nibbles are expanded to E4M3 bytes once per workgroup while staging
//       into LDS (v_perm lookup).  The scale product s_x[m] s_w[n] of all 32x32
//       pairs is one bf16 matrix instruction (outer product, exact in fp32),
//       so the per-group epilogue is a single fp32 FMA per element:
//       acc = fma(P_g, s_x s_w, acc).
// nvfp4 The E4M3 block scales have 4-bit mantissas, which no gfx950 block-scaled
//       instruction can apply (its scales are powers of two), and a per-16
//       epilogue would be VALU-bound.  Instead both operands are dequantized
//       exactly to fp16 (E2M1 x E4M3 needs 6 significant bits; range
//       2^-10..2688) with v_cvt_scalef32_pk_f16_fp4 + v_pk_mul_f16 and fed to
//       v_mfma_f32_32x32x16_f16 (K = 16 = one group): the scales ride inside
//       the operands and fp32 accumulation runs across all of K.  wtscale is
//       applied once at the end.
// Low-rank up: lora_act (fp32) is split into bf16 hi + lo and multiplied by
//       lora_up with bf16 matrix instructions accumulating into the same
//       registers (~16-bit accurate branch).
//
// PARTIALS=true is the parity export: the same staging, operand unpacking and
// matrix instructions, writing the exact per-group integer partials instead.

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kRowFp8 = 80;   // 64 E4M3 bytes + 16 pad (conflict-free 16-byte reads)
constexpr int kRowNib = 36;   // 32 nibble bytes + 4 pad

template <int PREC>
struct Stage;

template <>
struct Stage<kInt4> {
  uint8_t a[kBM * kRowFp8];
  uint8_t w[kBN * kRowFp8];
  uint16_t sa[kBM];
  uint16_t sw[kBN];
};

template <>
struct Stage<kNvfp4> {
  uint8_t a[kBM * kRowNib];
  uint8_t w[kBN * kRowNib];
  uint32_t sa[kBM];  // 4 E4M3 scale bytes (groups of this stage) per row
  uint32_t sw[kBN];
};

__device__ __forceinline__ bf16x8 scale_operand(uint16_t s, int h) {
  bf16x8 v = {};
  if (h == 0) v[0] = __builtin_bit_cast(__bf16, s);
  return v;
}

// E4M3 byte `sel` of a 32-bit word -> float (sel is a compile-time constant
// after unrolling).
__device__ __forceinline__ float e4m3_byte(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

__device__ __forceinline__ f16x8 dequant_e2m1_f16(uint32_t nib8, _Float16 scale) {
  f16x2 sc = {scale, scale};
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 0) * sc;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 1) * sc;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 2) * sc;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 3) * sc;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int PREC, int RB, bool PARTIALS>
__global__ __launch_bounds__(kThreads) void gemm_w4a4_lora_up_kernel(GemmArgs args) {
  __shared__ Stage<PREC> st[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = (int)args.M, K = (int)args.K, N = (int)args.N;
  const int K2 = K >> 1;
  const int m0 = blockIdx.x * kBM;
  const int n0 = blockIdx.y * kBN;
  const int nstages = K / kBK;
  const uint8_t* __restrict__ ac = (const uint8_t*)args.act_codes;
  const uint8_t* __restrict__ wc = (const uint8_t*)args.w_codes;

  // ---- global -> register prefetch assignment --------------------------------
  const int ld_row = tid >> 1;          // 0..127
  const int ld_half = tid & 1;          // which 16 bytes of the 32-byte slice
  const int a_row = min(m0 + ld_row, M - 1);
  const int w_row = min(n0 + ld_row, N - 1);
  const uint8_t* a_src = ac + (size_t)a_row * K2 + ld_half * 16;
  const uint8_t* w_src = wc + (size_t)w_row * K2 + ld_half * 16;
  const int sc_row = tid & 127;
  const bool sc_is_w = tid >= 128;
  u32x4 ra, rw;
  uint32_t rs;

  auto load_stage = [&](int s) {
    ra = *(const u32x4*)(a_src + s * 32);
    rw = *(const u32x4*)(w_src + s * 32);
    if constexpr (PREC == kInt4) {
      if (!PARTIALS) {
        const int G = K >> 6;
        const uint16_t* src = sc_is_w ? (const uint16_t*)args.w_scales + (size_t)min(n0 + sc_row, N - 1) * G
                                      : (const uint16_t*)args.act_scales + (size_t)min(m0 + sc_row, M - 1) * G;
        rs = src[s];
      }
    } else {
      if (!PARTIALS) {
        const int G = K >> 4;
        const uint8_t* src = sc_is_w ? (const uint8_t*)args.w_scales + (size_t)min(n0 + sc_row, N - 1) * G
                                     : (const uint8_t*)args.act_scales + (size_t)min(m0 + sc_row, M - 1) * G;
        rs = *(const uint32_t*)(src + s * 4);
      }
    }
  };

  auto store_stage = [&](int buf) {
    Stage<PREC>& S = st[buf];
    if constexpr (PREC == kInt4) {
      uint32_t ea[8], ew[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nibbles_to_e4m3(ra[i], kInt4LutLo, kInt4LutHi, ea[2 * i], ea[2 * i + 1]);
        nibbles_to_e4m3(rw[i], kInt4LutLo, kInt4LutHi, ew[2 * i], ew[2 * i + 1]);
      }
      uint8_t* pa = S.a + ld_row * kRowFp8 + ld_half * 32;
      uint8_t* pw = S.w + ld_row * kRowFp8 + ld_half * 32;
      *(u32x4*)(pa) = u32x4{ea[0], ea[1], ea[2], ea[3]};
      *(u32x4*)(pa + 16) = u32x4{ea[4], ea[5], ea[6], ea[7]};
      *(u32x4*)(pw) = u32x4{ew[0], ew[1], ew[2], ew[3]};
      *(u32x4*)(pw + 16) = u32x4{ew[4], ew[5], ew[6], ew[7]};
      if (!PARTIALS) {
        if (sc_is_w) S.sw[sc_row] = (uint16_t)rs;
        else S.sa[sc_row] = (uint16_t)rs;
      }
    } else {
      uint32_t* pa = (uint32_t*)(S.a + ld_row * kRowNib + ld_half * 16);
      uint32_t* pw = (uint32_t*)(S.w + ld_row * kRowNib + ld_half * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) { pa[i] = ra[i]; pw[i] = rw[i]; }
      if (!PARTIALS) {
        if (sc_is_w) S.sw[sc_row] = rs;
        else S.sa[sc_row] = rs;
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31;
  const int h = lane >> 5;
  const f32x16 zero16 = {};

  auto partial_store = [&](int i, int j, int g, int G, const f32x16& P, float mul) {
    const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
      if (row < M && col < N) args.partials[((size_t)row * N + col) * G + g] = (int32_t)(P[e] * mul);
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) load_stage(s + 1);
    const Stage<PREC>& S = st[buf];
    if constexpr (PREC == kInt4) {
      i32x8 aop[2], bop[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* p = S.a + (wm * 64 + i * 32 + l32) * kRowFp8 + h * 32;
        const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
        aop[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t* p = S.w + (wn * 64 + j * 32 + l32) * kRowFp8 + h * 32;
        const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
        bop[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      if constexpr (PARTIALS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[i], bop[j], zero16, 0, 0, 0, 127, 0, 127);
            partial_store(i, j, s, nstages, P, 1.0f);
          }
      } else {
        bf16x8 sop_a[2], sop_w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sop_a[i] = scale_operand(S.sa[wm * 64 + i * 32 + l32], h);
#pragma unroll
        for (int j = 0; j < 2; ++j) sop_w[j] = scale_operand(S.sw[wn * 64 + j * 32 + l32], h);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[i], bop[j], zero16, 0, 0, 0, 127, 0, 127);
            const f32x16 Sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sop_a[i], sop_w[j], zero16, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(P[e], Sc[e], acc[i][j][e]);
          }
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        f16x8 aop[2], bop[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rr = wm * 64 + i * 32 + l32;
          const uint32_t nib = *(const uint32_t*)(S.a + rr * kRowNib + gg * 8 + h * 4);
          _Float16 sc = (_Float16)1.0f;
          if (!PARTIALS) sc = (_Float16)e4m3_byte(S.sa[rr], gg);
          aop[i] = dequant_e2m1_f16(nib, sc);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cc = wn * 64 + j * 32 + l32;
          const uint32_t nib = *(const uint32_t*)(S.w + cc * kRowNib + gg * 8 + h * 4);
          _Float16 sc = (_Float16)1.0f;
          if (!PARTIALS) sc = (_Float16)e4m3_byte(S.sw[cc], gg);
          bop[j] = dequant_e2m1_f16(nib, sc);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if constexpr (PARTIALS) {
              const f32x16 D = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[j], zero16, 0, 0, 0);
              partial_store(i, j, s * 4 + gg, nstages * 4, D, 4.0f);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[j], acc[i][j], 0, 0, 0);
            }
          }
      }
    }
    if (s + 1 < nstages) store_stage(buf ^ 1);
    __syncthreads();
  }

  if constexpr (!PARTIALS) {
    if constexpr (PREC == kNvfp4) {
      const float t = args.wtscale;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = __fmul_rn(acc[i][j][e], t);
    }
    // ---- low-rank up: acc += (lora_act_hi + lora_act_lo) lora_up^T -----------
    if constexpr (RB > 0) {
      constexpr int rank = RB * 16;
      const uint16_t* __restrict__ lu = (const uint16_t*)args.lora_up;
#pragma unroll
      for (int rs = 0; rs < RB; ++rs) {
        bf16x8 ahi[2], alo[2], bo[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = min(m0 + wm * 64 + i * 32 + l32, M - 1);
          const float* la = args.lora_act + (size_t)row * rank + rs * 16 + h * 8;
          const f32x4 v0 = *(const f32x4*)la, v1 = *(const f32x4*)(la + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = e < 4 ? v0[e] : v1[e - 4];
            const __bf16 hb = (__bf16)v;
            ahi[i][e] = hb;
            alo[i][e] = (__bf16)(v - (float)hb);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = min(n0 + wn * 64 + j * 32 + l32, N - 1);
          bo[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(lu + (size_t)col * rank + rs * 16 + h * 8));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[i], bo[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[i], bo[j], acc[i][j], 0, 0, 0);
          }
      }
    }
    // ---- bias + bf16 store --------------------------------------------------
    const uint16_t* bias = (const uint16_t*)args.bias;
    uint16_t* out = (uint16_t*)args.out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
      const float bv = (bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
          if (row < M && col < N) out[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][e] + bv);
        }
    }
  }
}

template <int PREC, bool PARTIALS>
static hipError_t dispatch_rank(const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.M + kBM - 1) / kBM), (unsigned)((a.N + kBN - 1) / kBN));
  dim3 block(kThreads);
#define SVDQ_K2_CASE(rb)                                                                        \
  case rb:                                                                                      \
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, rb, PARTIALS>), grid, block, 0, s, a); \
    break;
  if (PARTIALS) {
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, 0, true>), grid, block, 0, s, a);
  } else {
    switch (a.rank / 16) {
      SVDQ_K2_CASE(0)
      SVDQ_K2_CASE(1)
      SVDQ_K2_CASE(2)
      SVDQ_K2_CASE(3)
      SVDQ_K2_CASE(4)
      SVDQ_K2_CASE(5)
      SVDQ_K2_CASE(6)
      SVDQ_K2_CASE(7)
      SVDQ_K2_CASE(8)
      default: return hipErrorInvalidValue;
    }
  }
#undef SVDQ_K2_CASE
  return hipGetLastError();
}

hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream) {
  const bool partials = a.partials != nullptr;
  if (a.precision == kInt4)
    return partials ? dispatch_rank<kInt4, true>(a, stream) : dispatch_rank<kInt4, false>(a, stream);
  return partials ? dispatch_rank<kNvfp4, true>(a, stream) : dispatch_rank<kNvfp4, false>(a, stream);
}

}  // namespace svdq
