// Kernel 2 of the SVDQ W4A4 linear: the 4-bit x 4-bit product with per-group
// scales, plus the low-rank up projection, the bias and the bf16 store.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table (svdq_w4a4:
// int4 with group 64 or nvfp4 with group 16, each with an SVDQ low-rank
// correction); bf16 compute dtype from the "NunchakuLiteQuantizationConfig"
// section.  Y = sum_g P_g * s_x * s_w * wtscale + lora_act lora_up^T + bias.
//
// gfx950 design
// -------------
// Workgroup tile 256 (M) x 192 (N) -- 256 workgroups for a 4096 x 3072
// output, one per CU -- with 8 waves (4 x 2), each wave 64 x 96 = 2 x 3 blocks
// of 32 x 32; 64 columns of K per stage.  Raw 4-bit codes are prefetched into
// registers, expanded cooperatively (each code once per workgroup) into a
// double-buffered LDS stage, and read back as matrix-instruction operands with
// conflict-free 16-byte LDS reads (padded rows).  Tiles are visited in groups
// of 4 M-tiles and mapped so the workgroups on one XCD share A and W tiles in
// that XCD's L2.
//
// int4  A group (64 k) is exactly one v_mfma_scale_f32_32x32x64_f8f6f4 with
//       E4M3 operands and unit block scales: the codes -7..7 are exact in E4M3,
//       so the fp32 result is the exact integer partial P_g.  Nibbles become
//       E4M3 bytes with a v_perm lookup: the activations already by the
//       quantize kernel (written once, in "expansion order"), the weights per
//       workgroup while staging, in the same order.  Per group the epilogue is
//       acc = fma(P_g, fl32(s_x[m] s_w[n]), acc) (s_x s_w is exact in fp32):
//       each lane holds one column and reads the four runs of four rows it
//       owns from an fp32 copy of s_x in LDS.  (Forming s_x s_w with a bf16
//       outer-product matrix instruction instead would save the multiply, but
//       the compiler then hoists those instructions and the 64 x 96 wave tile
//       no longer fits in 256 registers.)
// nvfp4 The E4M3 block scales have 4-bit mantissas, which the gfx950
//       block-scaled instructions cannot apply (their scales are powers of
//       two), and a per-16 epilogue would be VALU-bound.  Both operands are
//       dequantized exactly to fp16 while staging (E2M1 x E4M3 needs 6
//       significant bits, range 2^-10..2688) and v_mfma_f32_32x32x16_f16
//       (K = 16 = one group) accumulates across all of K in fp32; wtscale is
//       applied once at the end.
// Low-rank up: lora_act (fp32) split into bf16 hi + lo, times lora_up, with
//       bf16 matrix instructions accumulating into the same registers.
//
// PARTIALS=true is the parity export: the same staging, unpacking and matrix
// instructions, writing the exact per-group integer partials instead.

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int kBM = 256;
constexpr int kBN = 192;
constexpr int kBK = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWM = 4;   // waves along M
constexpr int kIB = 2;   // 32-row blocks per wave
constexpr int kJB = 3;   // 32-column blocks per wave
constexpr int kGroupM = 4;

template <int PREC>
struct alignas(16) Tile {
  // int4: 64 E4M3 bytes per row; nvfp4: 64 fp16 values per row; +16 bytes pad
  static constexpr int ROW = PREC == kInt4 ? 80 : 144;
  uint8_t a[kBM * ROW];
  uint8_t w[kBN * ROW];
  float sa[PREC == kInt4 ? kBM : 1];   // int4 group scales of this stage, as fp32
  float sw[PREC == kInt4 ? kBN : 1];
};

struct RawStage {
  u32x4 a, a2, w;       // A: 32 nibbles (a) or 32 E4M3 bytes (a, a2); W: 32 nibbles
  uint32_t sa, sw;      // int4: the row's group scale; nvfp4: two E4M3 bytes
};

__device__ __forceinline__ f16x8 dequant_e2m1_f16(uint32_t nib8, _Float16 scale) {
  const f16x2 sc = {scale, scale};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib8, 1.0f, 3) * sc;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Logical tile of this workgroup: consecutive workgroups land on different
// XCDs, so first gather the ids that share an XCD, then walk groups of
// kGroupM M-tiles column by column.
__device__ __forceinline__ void tile_of(int bid, int nmt, int nnt, int& mt, int& nt) {
  const int total = nmt * nnt;
  int logical = bid;
  if (total % 8 == 0) logical = (bid % 8) * (total / 8) + bid / 8;
  const int per_group = kGroupM * nnt;
  const int group = logical / per_group;
  const int first = group * kGroupM;
  const int gsize = min(nmt - first, kGroupM);
  const int r = logical - group * per_group;
  mt = first + r % gsize;
  nt = r / gsize;
}

template <int PREC, int RB, bool PARTIALS>
__global__ __launch_bounds__(kThreads) void gemm_w4a4_lora_up_kernel(GemmArgs args) {
  __shared__ Tile<PREC> st[2];
  constexpr int ROW = Tile<PREC>::ROW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % kWM, wn = wave / kWM;
  const int M = (int)args.M, K = (int)args.K, N = (int)args.N;
  const int K2 = K >> 1;
  const int nmt = (M + kBM - 1) / kBM, nnt = (N + kBN - 1) / kBN;
  int mt, nt;
  tile_of(blockIdx.x, nmt, nnt, mt, nt);
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int nstages = K / kBK;

  // ---- loader roles --------------------------------------------------------
  const int ld_row = tid >> 1;  // A: 0..255, W: 0..191 (threads < 384)
  const int ld_half = tid & 1;  // which 16 bytes (32 codes) of the 64-code stage
  const bool w_loader = tid < 2 * kBN;
  const int a_row = min(m0 + ld_row, M - 1);
  const int w_row = min(n0 + (w_loader ? ld_row : 0), N - 1);
  // int4 activations arrive as E4M3 bytes [M, K] from the quantize kernel
  // (except for the partials export, which takes packed nibbles)
  constexpr bool A_FP8 = PREC == kInt4 && !PARTIALS;
  const uint8_t* a_src = A_FP8 ? (const uint8_t*)args.act_codes + (size_t)a_row * K + ld_half * 32
                               : (const uint8_t*)args.act_codes + (size_t)a_row * K2 + ld_half * 16;
  const uint8_t* w_src = (const uint8_t*)args.w_codes + (size_t)w_row * K2 + ld_half * 16;

  auto load = [&](RawStage& r, int s) {
    if constexpr (A_FP8) {
      r.a = *(const u32x4*)(a_src + s * 64);
      r.a2 = *(const u32x4*)(a_src + s * 64 + 16);
    } else {
      r.a = *(const u32x4*)(a_src + s * 32);
    }
    if (w_loader) r.w = *(const u32x4*)(w_src + s * 32);
    if constexpr (!PARTIALS) {
      if constexpr (PREC == kInt4) {
        const int G = K >> 6;
        if (ld_half == 0) {
          r.sa = ((const uint16_t*)args.act_scales)[(size_t)a_row * G + s];
          if (w_loader) r.sw = ((const uint16_t*)args.w_scales)[(size_t)w_row * G + s];
        }
      } else {
        const int G = K >> 4;
        r.sa = *(const uint16_t*)((const uint8_t*)args.act_scales + (size_t)a_row * G + s * 4 + ld_half * 2);
        if (w_loader)
          r.sw = *(const uint16_t*)((const uint8_t*)args.w_scales + (size_t)w_row * G + s * 4 + ld_half * 2);
      }
    }
  };

  auto store = [&](Tile<PREC>& T, const RawStage& r) {
    if constexpr (PREC == kInt4) {
      uint32_t e[8];
      uint8_t* pa = T.a + ld_row * ROW + ld_half * 32;
      if constexpr (A_FP8) {
        *(u32x4*)(pa) = r.a;
        *(u32x4*)(pa + 16) = r.a2;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) nibbles_to_e4m3(r.a[i], kInt4LutLo, kInt4LutHi, e[2 * i], e[2 * i + 1]);
        *(u32x4*)(pa) = u32x4{e[0], e[1], e[2], e[3]};
        *(u32x4*)(pa + 16) = u32x4{e[4], e[5], e[6], e[7]};
      }
      if (w_loader) {
#pragma unroll
        for (int i = 0; i < 4; ++i) nibbles_to_e4m3(r.w[i], kInt4LutLo, kInt4LutHi, e[2 * i], e[2 * i + 1]);
        uint8_t* pw = T.w + ld_row * ROW + ld_half * 32;
        *(u32x4*)(pw) = u32x4{e[0], e[1], e[2], e[3]};
        *(u32x4*)(pw + 16) = u32x4{e[4], e[5], e[6], e[7]};
      }
      if (!PARTIALS && ld_half == 0) {
        T.sa[ld_row] = bf16_bits_to_f32((uint16_t)r.sa);
        if (w_loader) T.sw[ld_row] = bf16_bits_to_f32((uint16_t)r.sw);
      }
    } else {
      // nvfp4: 32 codes = two groups of 16; dequantize exactly to fp16
      _Float16 sa0 = (_Float16)1.0f, sa1 = (_Float16)1.0f, sw0 = (_Float16)1.0f, sw1 = (_Float16)1.0f;
      if constexpr (!PARTIALS) {
        sa0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sa, 0);
        sa1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sa, 1);
        sw0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sw, 0);
        sw1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sw, 1);
      }
      uint8_t* pa = T.a + ld_row * ROW + ld_half * 64;
      *(f16x8*)(pa) = dequant_e2m1_f16(r.a[0], sa0);
      *(f16x8*)(pa + 16) = dequant_e2m1_f16(r.a[1], sa0);
      *(f16x8*)(pa + 32) = dequant_e2m1_f16(r.a[2], sa1);
      *(f16x8*)(pa + 48) = dequant_e2m1_f16(r.a[3], sa1);
      if (w_loader) {
        uint8_t* pw = T.w + ld_row * ROW + ld_half * 64;
        *(f16x8*)(pw) = dequant_e2m1_f16(r.w[0], sw0);
        *(f16x8*)(pw + 16) = dequant_e2m1_f16(r.w[1], sw0);
        *(f16x8*)(pw + 32) = dequant_e2m1_f16(r.w[2], sw1);
        *(f16x8*)(pw + 48) = dequant_e2m1_f16(r.w[3], sw1);
      }
    }
  };

  f32x16 acc[kIB][kJB];
#pragma unroll
  for (int i = 0; i < kIB; ++i)
#pragma unroll
    for (int j = 0; j < kJB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31;
  const int h = lane >> 5;
  const f32x16 zero16 = {};

  auto partial_store = [&](int i, int j, int g, int G, const f32x16& P, float mul) {
    const int col = n0 + wn * (kJB * 32) + j * 32 + l32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + wm * (kIB * 32) + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
      if (row < M && col < N) args.partials[((size_t)row * N + col) * G + g] = (int32_t)(P[e] * mul);
    }
  };

  auto compute = [&](const Tile<PREC>& T, int s) {
    if constexpr (PREC == kInt4) {
      i32x8 aop[kIB];
#pragma unroll
      for (int i = 0; i < kIB; ++i) {
        const uint8_t* p = T.a + (wm * (kIB * 32) + i * 32 + l32) * ROW + h * 32;
        const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
        aop[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        const uint8_t* p = T.w + (wn * (kJB * 32) + j * 32 + l32) * ROW + h * 32;
        const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
        const i32x8 bop = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const float swf = PARTIALS ? 0.f : T.sw[wn * (kJB * 32) + j * 32 + l32];
#pragma unroll
        for (int i = 0; i < kIB; ++i) {
          const f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[i], bop, zero16, 0, 0, 0, 127, 0, 127);
          if constexpr (PARTIALS) {
            partial_store(i, j, s, nstages, P, 1.0f);
          } else {
            // rows of this lane: 8 q4 + 4 h + (0..3), q4 = 0..3
            const float* rowp = T.sa + wm * (kIB * 32) + i * 32 + h * 4;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 s4 = *(const f32x4*)(rowp + q4 * 8);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[i][j][q4 * 4 + e] = __builtin_fmaf(P[q4 * 4 + e], __fmul_rn(s4[e], swf), acc[i][j][q4 * 4 + e]);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        f16x8 aop[kIB], bop[kJB];
#pragma unroll
        for (int i = 0; i < kIB; ++i)
          aop[i] = *(const f16x8*)(T.a + (wm * (kIB * 32) + i * 32 + l32) * ROW + gg * 32 + h * 16);
#pragma unroll
        for (int j = 0; j < kJB; ++j)
          bop[j] = *(const f16x8*)(T.w + (wn * (kJB * 32) + j * 32 + l32) * ROW + gg * 32 + h * 16);
#pragma unroll
        for (int i = 0; i < kIB; ++i)
#pragma unroll
          for (int j = 0; j < kJB; ++j) {
            if constexpr (PARTIALS) {
              const f32x16 D = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[j], zero16, 0, 0, 0);
              partial_store(i, j, s * 4 + gg, nstages * 4, D, 4.0f);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[j], acc[i][j], 0, 0, 0);
            }
          }
      }
    }
  };

  // ---- main loop -------------------------------------------------------------
  // The registers of stage s+1 are loaded right after the barrier that ends
  // stage s-1 and written to LDS after the compute of stage s, so a whole
  // compute hides their latency (loading them at the top of the same
  // iteration lets the compiler wait for them before the compute).
  RawStage r0;
  load(r0, 0);
  store(st[0], r0);
  __syncthreads();
  if (nstages > 1) load(r0, 1);
  for (int s = 0; s < nstages; ++s) {
    compute(st[s & 1], s);
    if (s + 1 < nstages) store(st[(s + 1) & 1], r0);
    __syncthreads();
    if (s + 2 < nstages) load(r0, s + 2);
  }

  if constexpr (!PARTIALS) {
    if constexpr (PREC == kNvfp4) {
      const float t = args.wtscale;
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int j = 0; j < kJB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = __fmul_rn(acc[i][j][e], t);
    }
    // ---- low-rank up: acc += (lora_act_hi + lora_act_lo) lora_up^T -----------
    if constexpr (RB > 0) {
      constexpr int rank = RB * 16;
      const uint16_t* __restrict__ lu = (const uint16_t*)args.lora_up;
#pragma unroll
      for (int rs = 0; rs < RB; ++rs) {
        bf16x8 ahi[kIB], alo[kIB], bo[kJB];
#pragma unroll
        for (int i = 0; i < kIB; ++i) {
          const int row = min(m0 + wm * (kIB * 32) + i * 32 + l32, M - 1);
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
        for (int j = 0; j < kJB; ++j) {
          const int col = min(n0 + wn * (kJB * 32) + j * 32 + l32, N - 1);
          bo[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(lu + (size_t)col * rank + rs * 16 + h * 8));
        }
#pragma unroll
        for (int i = 0; i < kIB; ++i)
#pragma unroll
          for (int j = 0; j < kJB; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[i], bo[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[i], bo[j], acc[i][j], 0, 0, 0);
          }
      }
    }
    // ---- bias + bf16 store --------------------------------------------------
    const uint16_t* bias = (const uint16_t*)args.bias;
    uint16_t* out = (uint16_t*)args.out;
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      const int col = n0 + wn * (kJB * 32) + j * 32 + l32;
      const float bv = (bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * (kIB * 32) + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
          if (row < M && col < N) out[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][e] + bv);
        }
    }
  }
}

template <int PREC, bool PARTIALS>
static hipError_t dispatch_rank(const GemmArgs& a, hipStream_t s) {
  const unsigned tiles = (unsigned)(((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN));
  dim3 grid(tiles), block(kThreads);
  if constexpr (PARTIALS) {
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, 0, true>), grid, block, 0, s, a);
  } else {
#define SVDQ_K2_CASE(rb)                                                                     \
  case rb:                                                                                   \
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, rb, false>), grid, block, 0, s, a); \
    break;
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
#undef SVDQ_K2_CASE
  }
  return hipGetLastError();
}

hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream) {
  const bool partials = a.partials != nullptr;
  if (a.precision == kInt4)
    return partials ? dispatch_rank<kInt4, true>(a, stream) : dispatch_rank<kInt4, false>(a, stream);
  return partials ? dispatch_rank<kNvfp4, true>(a, stream) : dispatch_rank<kNvfp4, false>(a, stream);
}

}  // namespace svdq
