// Kernel 2 of the SVDQ W4A4 linear: the 4-bit x 4-bit product with per-group
// scales, plus the low-rank up projection, the bias and the bf16 store.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table (svdq_w4a4:
// int4 with group 64 or nvfp4 with group 16, each with an SVDQ low-rank
// correction); bf16 compute dtype from the "NunchakuLiteQuantizationConfig"
// section.  Y = sum_g P_g * s_x * s_w * wtscale + lora_act lora_up^T + bias,
// P_g the integer dot product of the codes of group g.
//
// gfx950 design
// -------------
// The group scales are folded into the operands instead of being applied to
// every output once per group.  A code times its group scale needs at most
// 3 + 8 significant bits (int4 |q| <= 7 times a bf16 scale) or 2 + 4 (E2M1
// times E4M3), so both operands are exact fp16 values and one fp16 matrix
// product with fp32 accumulation over all of K gives sum_g s_x s_w P_g with
// exact products:
//   A  the quantize kernel already writes q * s_x (nvfp4: e2m1 * dec(s8)) as
//      fp16; int4 rows carry a power of two 2^-E[m] so that they fit fp16,
//      undone here after the product (row_scale);
//   W  converted while staging: codes via a v_perm table into fp16, times the
//      group scale (int4: times 2^-F[n], one power of two per weight row chosen
//      from its largest scale, undone at the end; nvfp4: dec(s8), with
//      wtscale applied at the end).
// A per-group fp32 epilogue (two VALU operations per output and group) would
// outweigh the matrix work; with folded scales the main loop is matrix
// instructions, LDS traffic and the staging of W.
//
// Workgroup tile 256 (M) x 192 (N) -- 256 workgroups for a 4096 x 3072
// output, one per CU -- with 8 waves (4 x 2), each wave 64 x 96 = 2 x 3 blocks
// of 32 x 32; 64 columns of K per stage, v_mfma_f32_32x32x16_f16.  Raw stages
// are loaded two stages ahead into registers and written to a double-buffered
// LDS stage (padded rows: conflict-free 16-byte reads).  Tiles are visited in
// groups of 4 M-tiles, mapped so that the workgroups on one XCD share A and W
// tiles in its L2.
// Low-rank up: lora_act (fp32) split into bf16 hi + lo, times lora_up, with
// bf16 matrix instructions accumulating into the same registers.
//
// PARTIALS=true is the parity export: the same staging and matrix
// instructions with unit scales (A from packed codes), writing the exact
// per-group integer partials (nvfp4: doubled E2M1 codes) instead.

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
constexpr int kRow = 144;  // LDS bytes per staged row: 64 fp16 + 16 pad
constexpr int kMaxScaleG = 64;  // int4 weight-scale table in LDS for K <= 4096

struct alignas(16) Stage {
  uint8_t a[kBM * kRow];
  uint8_t w[kBN * kRow];
};

// One stage of raw operands in registers.  Every thread has the same role:
// A piece i (0..3) = 16 bytes of fp16 (linear) or 4 bytes of codes (partials)
// holding columns 8c..8c+7 (c = tid % 8) of tile row tid/8 + 64 i; W piece j
// (0..2) = 4 bytes of codes for columns 8c..8c+7 of tile row tid/8 + 64 j.  A
// load instruction therefore covers whole 128-byte (A) or 32-byte (W) row
// slices of 8 rows, and the staging code has no per-wave branches.
struct RawStage {
  u32x4 a[4];
  uint32_t w[3];
  uint32_t sw[3];  // nvfp4: the E4M3 scale byte of each W piece (int4 reads a table)
};

// Raw buffer descriptor over `bytes` bytes at p (sizes past 2^31 - 1 are
// clamped: a tile never addresses that far from its base).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, size_t bytes) {
  const int n = bytes > 0x7fffffffu ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
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

// WT (int4 only, K <= 64 kMaxScaleG): the weight group scales come from a
// table in LDS filled once per workgroup instead of one load per row and stage.
template <int PREC, int RB, bool PARTIALS, bool WT>
__global__ __launch_bounds__(kThreads) void gemm_w4a4_lora_up_kernel(GemmArgs args) {
  __shared__ Stage st[2];
  __shared__ float wexp[kBN];   // int4: 2^F[n] of this tile's weight rows
  __shared__ float wdown[kBN];  // int4: 2^-F[n]
  __shared__ _Float16 wsc[WT ? kBN * kMaxScaleG : 1];  // int4: s_w * 2^-F[n]
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
  constexpr bool kRowExp = PREC == kInt4 && !PARTIALS;

  // ---- loader roles --------------------------------------------------------
  // Buffer loads: one descriptor per operand based at this tile's first row,
  // 32-bit lane offsets, the stage offset in a scalar register.  Rows past
  // the end of the matrix lie beyond the descriptor's size and read as zero.
  const int lc = tid & 7;    // column chunk: columns 8 lc .. 8 lc + 7 of the stage
  const int lr = tid >> 3;   // tile row of piece 0 (piece i: lr + 64 i)
  const size_t a_row_bytes = PARTIALS ? (size_t)K2 : (size_t)K * 2;
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc((const uint8_t*)args.act + (size_t)m0 * a_row_bytes,
                                                (size_t)(M - m0) * a_row_bytes);
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc((const uint8_t*)args.w_codes + (size_t)n0 * K2,
                                                (size_t)(N - n0) * K2);
  const size_t ws_row_bytes = PREC == kInt4 ? (size_t)(K >> 6) * 2 : (size_t)(K >> 4);
  const __amdgpu_buffer_rsrc_t ws_rs = make_rsrc((const uint8_t*)args.w_scales + (size_t)n0 * ws_row_bytes,
                                                 PARTIALS ? 0 : (size_t)(N - n0) * ws_row_bytes);
  int a_off[4], w_off[3], ws_off[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_off[i] = (lr + 64 * i) * (int)a_row_bytes + lc * (PARTIALS ? 4 : 16);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    w_off[j] = (lr + 64 * j) * K2 + lc * 4;
    ws_off[j] = (lr + 64 * j) * (int)ws_row_bytes + (PREC == kNvfp4 ? (lc >> 1) : 0);
  }

  // int4: per weight row the power of two 2^-F that makes every q * s_w * 2^-F
  // an exact fp16 (from the row's largest group scale); for K <= 4096 the
  // scaled group scales s_w * 2^-F themselves go to an LDS table, read here
  // with whole-row loads instead of one scattered load per row and stage
  const int G64 = K >> 6;
  if constexpr (kRowExp) {
    if (tid < kBN) {
      // the row's scales, two per load (G64 is even: rows are 4-byte aligned)
      const uint16_t* srow = (const uint16_t*)args.w_scales + (size_t)min(n0 + tid, N - 1) * G64;
      float m = 0.f;
      if constexpr (WT) {
        uint32_t v[kMaxScaleG / 2];  // all of them in flight at once, kept for the table
#pragma unroll
        for (int p = 0; p < kMaxScaleG / 2; ++p)
          if (2 * p < G64) v[p] = *(const uint32_t*)(srow + 2 * p);
#pragma unroll
        for (int p = 0; p < kMaxScaleG / 2; ++p)
          if (2 * p < G64) m = fmaxf(m, fmaxf(bf16_lo(v[p]), bf16_hi(v[p])));
        const int F = m > 0.f ? fp16_fit_exponent(m) : 0;
        wexp[tid] = __builtin_ldexpf(1.0f, F);
        const float down = __builtin_ldexpf(1.0f, -F);
        wdown[tid] = down;
#pragma unroll
        for (int p = 0; p < kMaxScaleG / 2; ++p)
          if (2 * p < G64) {
            wsc[tid * kMaxScaleG + 2 * p] = (_Float16)(bf16_lo(v[p]) * down);
            wsc[tid * kMaxScaleG + 2 * p + 1] = (_Float16)(bf16_hi(v[p]) * down);
          }
      } else {
        for (int g0 = 0; g0 < G64; g0 += 16) {
          uint32_t v[8];
#pragma unroll
          for (int p = 0; p < 8; ++p)
            if (g0 + 2 * p < G64) v[p] = *(const uint32_t*)(srow + g0 + 2 * p);
#pragma unroll
          for (int p = 0; p < 8; ++p)
            if (g0 + 2 * p < G64) m = fmaxf(m, fmaxf(bf16_lo(v[p]), bf16_hi(v[p])));
        }
        const int F = m > 0.f ? fp16_fit_exponent(m) : 0;
        wexp[tid] = __builtin_ldexpf(1.0f, F);
        wdown[tid] = __builtin_ldexpf(1.0f, -F);
      }
    }
    __syncthreads();
  }

  auto load = [&](RawStage& r, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (PARTIALS) r.a[i][0] = __builtin_amdgcn_raw_buffer_load_b32(a_rs, a_off[i], s * 32, 0);
      else r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off[i], s * 128, 0);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      r.w[j] = __builtin_amdgcn_raw_buffer_load_b32(w_rs, w_off[j], s * 32, 0);
      if constexpr (PREC == kNvfp4 && !PARTIALS) r.sw[j] = __builtin_amdgcn_raw_buffer_load_b8(ws_rs, ws_off[j], s * 4, 0);
      if constexpr (PREC == kInt4 && !PARTIALS && !WT)
        r.sw[j] = __builtin_amdgcn_raw_buffer_load_b16(ws_rs, ws_off[j], s * 2, 0);
    }
  };

  // staging of one raw stage in four parts (A piece i and W piece i), so that
  // it can be interleaved with the matrix instructions of the previous stage
  auto store_part = [&](Stage& T, const RawStage& r, int i, int s) {
    uint8_t* pa = T.a + (lr + 64 * i) * kRow + lc * 16;
    if constexpr (PARTIALS) {
      // unit scales; nvfp4 doubles the E2M1 codes so that they are integers
      const _Float16 one = (_Float16)(PREC == kInt4 ? 1.0f : 2.0f);
      *(f16x8*)pa = PREC == kInt4 ? int4x8_to_f16_scaled(r.a[i][0], one) : e2m1x8_to_f16_scaled(r.a[i][0], one);
    } else {
      *(u32x4*)pa = r.a[i];
    }
    if (i < 3) {
      const int wrow = lr + 64 * i;
      uint8_t* pw = T.w + wrow * kRow + lc * 16;
      _Float16 sc = (_Float16)(PREC == kInt4 ? 1.0f : 2.0f);
      if constexpr (!PARTIALS) {
        if constexpr (PREC == kInt4) {
          if constexpr (WT) sc = wsc[wrow * kMaxScaleG + s];
          else sc = (_Float16)(bf16_bits_to_f32((uint16_t)r.sw[i]) * wdown[wrow]);  // exact: a power of two
        } else {
          sc = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sw[i], 0);
        }
      }
      *(f16x8*)pw = PREC == kInt4 ? int4x8_to_f16_scaled(r.w[i], sc) : e2m1x8_to_f16_scaled(r.w[i], sc);
    }
  };
  auto store = [&](Stage& T, const RawStage& r, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store_part(T, r, i, s);
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

  // exact integer partials of one group (fp32 holds them exactly)
  auto partial_store = [&](int g, int G) {
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        const int col = n0 + wn * (kJB * 32) + j * 32 + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * (kIB * 32) + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
          if (row < M && col < N) args.partials[((size_t)row * N + col) * G + g] = (int32_t)acc[i][j][e];
          acc[i][j][e] = 0.f;
        }
      }
  };

  // one stage: 4 k steps of 16, each 2 A and 3 W operand reads and 6 products.
  // The operands of k step ks+1 are read before the products of step ks are
  // issued (two register sets); with `nxt`, part ks of the next stage is
  // staged among the products of step ks (its VALU work and LDS writes issue
  // while the matrix instructions execute).
  auto compute = [&](const Stage& T, int s, Stage* nxt, const RawStage* r) {
    f16x8 aop[2][kIB], bop[2][kJB];
    auto rd = [&](int ks, f16x8* ao, f16x8* bo) {
#pragma unroll
      for (int i = 0; i < kIB; ++i)
        ao[i] = *(const f16x8*)(T.a + (wm * (kIB * 32) + i * 32 + l32) * kRow + ks * 32 + h * 16);
#pragma unroll
      for (int j = 0; j < kJB; ++j)
        bo[j] = *(const f16x8*)(T.w + (wn * (kJB * 32) + j * 32 + l32) * kRow + ks * 32 + h * 16);
    };
    rd(0, aop[0], bop[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) rd(ks + 1, aop[(ks + 1) & 1], bop[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int j = 0; j < kJB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[ks & 1][i], bop[ks & 1][j], acc[i][j], 0, 0, 0);
      if (nxt) store_part(*nxt, *r, ks, s + 1);
      if constexpr (!PARTIALS) {
        // order: next operands' LDS reads, then products interleaved with the
        // staging arithmetic, then the staging LDS writes
        if (ks < 3) __builtin_amdgcn_sched_group_barrier(0x100, kIB + kJB, 0);
#pragma unroll
        for (int m = 0; m < kIB * kJB; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
      }
      if constexpr (PARTIALS && PREC == kNvfp4) partial_store(s * 4 + ks, nstages * 4);
    }
    if constexpr (PARTIALS && PREC == kInt4) partial_store(s, nstages);
  };

  // ---- main loop -------------------------------------------------------------
  // Two raw stages in registers: the one for stage s+1 is staged into LDS in
  // parts among the k steps of stage s, and its slot is refilled with stage
  // s+3 right after the barrier, so each load has two stages of compute to
  // arrive.  The steady state is straight-line code (no conditions), so the
  // staging can be scheduled among the matrix instructions; it is unrolled
  // by two so that every register array index is a compile-time constant (a
  // runtime index would move the array to scratch).
  RawStage r0, r1;
  load(r0, 0);
  if (nstages > 1) load(r1, 1);
  store(st[0], r0, 0);
  lds_barrier();
  if (nstages > 2) load(r0, 2);
  int s = 0;
  for (; s + 4 < nstages; s += 2) {
    compute(st[0], s, &st[1], &r1);
    lds_barrier();
    load(r1, s + 3);
    compute(st[1], s + 1, &st[0], &r0);
    lds_barrier();
    load(r0, s + 4);
  }
  for (; s < nstages; s += 2) {  // the last (at most four) stages
    compute(st[0], s, s + 1 < nstages ? &st[1] : nullptr, &r1);
    lds_barrier();
    if (s + 3 < nstages) load(r1, s + 3);
    if (s + 1 < nstages) {
      compute(st[1], s + 1, s + 2 < nstages ? &st[0] : nullptr, &r0);
      lds_barrier();
      if (s + 4 < nstages) load(r0, s + 4);
    }
  }

  if constexpr (!PARTIALS) {
    // ---- undo the operand powers of two / apply the tensor scale -------------
    if constexpr (PREC == kInt4) {
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = min(m0 + wm * (kIB * 32) + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3), M - 1);
          const float ra = args.row_scale[row];
#pragma unroll
          for (int j = 0; j < kJB; ++j)
            acc[i][j][e] = __fmul_rn(acc[i][j][e], __fmul_rn(ra, wexp[wn * (kJB * 32) + j * 32 + l32]));
        }
    } else {
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
      for (int rs16 = 0; rs16 < RB; ++rs16) {
        bf16x8 ahi[kIB], alo[kIB], bo[kJB];
#pragma unroll
        for (int i = 0; i < kIB; ++i) {
          const int row = min(m0 + wm * (kIB * 32) + i * 32 + l32, M - 1);
          const float* la = args.lora_act + (size_t)row * rank + rs16 * 16 + h * 8;
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
          bo[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(lu + (size_t)col * rank + rs16 * 16 + h * 8));
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

template <int PREC, bool PARTIALS, bool WT>
static hipError_t dispatch_rank(const GemmArgs& a, hipStream_t s) {
  const unsigned tiles = (unsigned)(((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN));
  dim3 grid(tiles), block(kThreads);
  if constexpr (PARTIALS) {
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, 0, true, false>), grid, block, 0, s, a);
  } else {
#define SVDQ_K2_CASE(rb)                                                                     \
  case rb:                                                                                   \
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, rb, false, WT>), grid, block, 0, s, a); \
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
  if (a.precision == kInt4) {
    if (partials) return dispatch_rank<kInt4, true, false>(a, stream);
    return a.K / 64 <= kMaxScaleG ? dispatch_rank<kInt4, false, true>(a, stream)
                                  : dispatch_rank<kInt4, false, false>(a, stream);
  }
  return partials ? dispatch_rank<kNvfp4, true, false>(a, stream) : dispatch_rank<kNvfp4, false, false>(a, stream);
}

}  // namespace svdq
