// AWQ W4A16 linear for the small-M adaptive-norm layers.
//
// Method: Nunchaku Lite pages, "Supported quantization types" table, row
// awq_w4a16 (int4 weight-only, group 64); the news article assigns this path to
// the precision-sensitive adaptive-normalization layers.  Reading of the
// format: unsigned codes q (0..15), per-group bf16 scale s and integer
// zero-point z, W = (q - z) s;  Y = X W^T + bias with fp32 accumulation.
//
// gfx950 design -- bandwidth-bound: 4.5 bits per weight streamed once per MT
// rows of X (MT = 2, 4 or 16; one token runs in the 2-row tile, whose second
// row is never stored).
// * A workgroup owns 32 weight rows (output columns) and MT rows of X; its 4
//   waves split K into four contiguous group ranges.  The workgroup first
//   builds its (s, -s (128 + z)) table in LDS.
// * Each wave streams its range in steps of 4 groups, with coalesced loads
//   (lane l: 16 bytes of weight rows l/8 + 8j, so each row contributes 128
//   contiguous bytes per instruction; non-temporal, the weights are read
//   once), and moves every step into its own LDS rows in the layout the
//   matrix instruction reads.  The loads of step s + 1 are issued as soon as
//   step s is in LDS, before its products: one step in flight per wave.
//   Deeper prefetch measured slower -- more bytes in flight lengthen every
//   load's latency, and a step's products wait for its data either way.
// * Matrix instruction 16x16x32 bf16 (D = 16 rows of X x 16 weight rows): it
//   consumes 512 weights per 4 passes, half the matrix-core time of the 32x32
//   shape per weight, which matters at M <= 16 where most of D is padding.
//   Lane (c = lane%16, kq = lane/16) holds, per group and 32-wide k step s,
//   the k values 16 kq + 8 s + 0..7 of weight row c (4 code bytes, so one
//   8-byte LDS read covers a group) and the same k of X row c.
// * Codes become bf16 operands 128 + q (0x4300 | q is the bit pattern of
//   128 + q) with one v_perm and one OR per pair.  A second operand holds 1
//   in every slot, so a third product collects sum_k x over the group, and
//   sum_k x (q - z) s = s sum_k x (128 + q) - s (128 + z) sum_k x: exact bf16
//   products, fp32 sums, two FMAs per output and group.
// * Rows of X beyond M read row M - 1 (each output row depends on its own X
//   row only, and rows beyond M are never stored).  The four K-range partials
//   are summed in LDS in a fixed order.

#include "device_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace svdq {

constexpr int kAwqWaves = 4;       // K ranges per workgroup
constexpr int kAwqStepG = 4;       // groups per step: 128 contiguous bytes of each weight row
constexpr int kAwqRowPitch = 144;  // LDS bytes per staged weight row (128 + 16 pad)
constexpr int kAwqXPitch = 528;    // LDS bytes per staged X row (256 bf16 + 16 pad)

// Operand order within every 8 consecutive k: {0, 2, 4, 6, 1, 3, 5, 7}.  Codes
// reach it with one v_perm per pair of codes (bytes 0x43 from a constant
// give the bf16 pattern 0x4300 | q of 128 + q); X is put in the same order
// once, when a step of X is staged in LDS.
__device__ __forceinline__ bf16x8 awq_operand(uint32_t w) {
  constexpr uint32_t kHi = 0x43434343u;
  const uint32_t lo = w & 0x0F0F0F0Fu;          // codes k0, k2, k4, k6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes k1, k3, k5, k7
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(kHi, lo, 0x04010400u);  // (k0, k2)
  r[1] = __builtin_amdgcn_perm(kHi, lo, 0x04030402u);  // (k4, k6)
  r[2] = __builtin_amdgcn_perm(kHi, hi, 0x04010400u);  // (k1, k3)
  r[3] = __builtin_amdgcn_perm(kHi, hi, 0x04030402u);  // (k5, k7)
  return __builtin_bit_cast(bf16x8, r);
}

// 8 bf16 of X in k order (pairs (0,1) (2,3) (4,5) (6,7)) -> operand order
__device__ __forceinline__ u32x4 awq_x_order(u32x4 v) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);  // (x0, x2)
  r[1] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);  // (x4, x6)
  r[2] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);  // (x1, x3)
  r[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);  // (x5, x7)
  return r;
}

// MT: rows of X per workgroup (2, 4 or 16); D: steps in flight per wave.
//
// Dynamic LDS: the workgroup's scale table float2 [32 rows][G + 2] holding
// (s, -s (128 + z)) per weight row and group, then per wave a staged step of
// codes [32 rows][kAwqRowPitch] and of X [MT rows][kAwqXPitch].
template <int MT, int D, bool WIDE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT == 16 ? 2 : 3, 3)))
void awq_w4a16_kernel(AwqArgs args) {
  static_assert(MT % 2 == 0, "X rows are loaded in pairs");
  constexpr int XV = MT / 2;  // 16-byte X loads per lane and step
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float part[kAwqWaves][16][33];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = (int)args.M, K = (int)args.K, N = (int)args.N;
  const int G = K >> 6;
  const int K2 = K >> 1;
  const int m0 = blockIdx.y * MT;
  const int rows = min(MT, M - m0);
  const int n0 = blockIdx.x * 32;

  float2* stab = (float2*)smem;
  const int G2 = G + 2;  // scale-table row pitch in float2: 400 bytes at G = 48, so the 16
                        // rows one read covers fall on different banks
  uint8_t* ws = smem + (size_t)32 * G2 * 8 + (size_t)wave * (32 * kAwqRowPitch + MT * kAwqXPitch);
  uint8_t* xs = ws + 32 * kAwqRowPitch;

  const int c = lane & 15;
  const int kq = lane >> 4;
  // this wave's contiguous range of groups, whole steps except at the end of K
  const int gpw = kAwqStepG * ((G + kAwqStepG * kAwqWaves - 1) / (kAwqStepG * kAwqWaves));
  const int g0 = min(G, wave * gpw);
  const int g1 = min(G, g0 + gpw);
  const int nsteps = (g1 - g0 + kAwqStepG - 1) / kAwqStepG;

  // ---- scale table: item (row r, group pair p) for r < 32, p < G/2 ----------
  const uint32_t* s32 = (const uint32_t*)args.scales + (size_t)n0 * (G / 2);
  const uint32_t* z32 = (const uint32_t*)args.zeros + (size_t)n0 * (G / 2);
  const int items = 16 * G;  // 32 rows x G/2 pairs, contiguous in both tables
  uint32_t sraw[4], zraw[4];
  auto load_items = [&](int base) {  // unconditional (clamped) loads keep the wait counts exact
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = min(base + tid + 256 * u, items - 1);
      sraw[u] = s32[it];
      zraw[u] = z32[it];
    }
  };
  // (s, -s (128 + z)) per row and group; both factors of the product are
  // exact (8-bit significands), so the fp32 product is exact
  auto store_items = [&](int base) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = base + tid + 256 * u;
      if (it < items) {
        const float sl = bf16_lo(sraw[u]), sh = bf16_hi(sraw[u]);
        const float zl = bf16_lo(zraw[u]), zh = bf16_hi(zraw[u]);
        const int row = it / (G / 2), pr = it - row * (G / 2);
        *(float4*)(stab + row * G2 + 2 * pr) = float4{sl, -sl * (128.0f + zl), sh, -sh * (128.0f + zh)};
      }
    }
  };
  load_items(0);

  // codes: lane l streams 16 bytes (half of group (l%8)/2 of the step) of
  // weight rows n0 + l/8 + 8j, j = 0..3 -- 128 contiguous bytes per row
  const int q8 = lane & 7;
  const uint8_t* wstream = (const uint8_t*)args.w_codes + (size_t)(n0 + (lane >> 3)) * K2 + (q8 & 1) * 16;
  // X: MT rows x 256 k of the step; load v covers rows 2v + l/32, k 8 (l%32)
  // .. +7.  Rows beyond M read row M - 1.
  const uint16_t* xbase = (const uint16_t*)args.x + (size_t)m0 * K;

  // D steps in flight; all loads of a step (codes and X) are issued together,
  // so the in-order memory counter releases whole steps.  Past the wave's
  // range (a partial last step, or the prologue of a short range) the loads
  // re-read the last valid group.
  u32x4 wr[D][4];
  u32x4 xr[D][XV];
  auto issue = [&](int slot, int step) {
    const int gs = g0 + step * kAwqStepG;
    const int gw = min(gs + (q8 >> 1), g1 - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wr[slot][j] = __builtin_nontemporal_load((const u32x4*)(wstream + (size_t)(8 * j) * K2 + (size_t)gw * 32));
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int r = min(2 * v + (lane >> 5), rows - 1);
      const int g = min(gs + ((lane & 31) >> 3), g1 - 1);
      xr[slot][v] = *(const u32x4*)(xbase + (size_t)r * K + (size_t)g * 64 + (lane & 7) * 8);
    }
  };
  // always in bounds (clamped to the last group), so issued unconditionally:
  // straight-line code keeps the compiler's memory-counter waits exact
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);

  store_items(0);
  if constexpr (WIDE) {  // K > 4096: the table takes more than one batch
    for (int base = 1024; base < items; base += 1024) {
      load_items(base);
      store_items(base);
    }
  }
  lds_barrier();  // the code and X prefetches stay in flight

  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  f32x4 accA = {}, accB = {};
  auto group = [&](int g, int i) {
    const f32x4 zero4 = {};
    // operands from this wave's LDS rows: codes 8 bytes of rows c and 16 + c,
    // X 32 bytes of row min(c, MT - 1)
    const u32x2 wa = *(const u32x2*)(ws + c * kAwqRowPitch + i * 32 + kq * 8);
    const u32x2 wb = *(const u32x2*)(ws + (16 + c) * kAwqRowPitch + i * 32 + kq * 8);
    const uint8_t* xp = xs + min(c, MT - 1) * kAwqXPitch + i * 128 + kq * 32;
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, *(const u32x4*)xp);
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xp + 16));
    const float2 pa = stab[c * G2 + g];
    const float2 pb = stab[(16 + c) * G2 + g];
    // k step 0 uses code bytes 0..3 (k = 16 kq + 0..7), step 1 bytes 4..7
    f32x4 tA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, awq_operand(wa[0]), zero4, 0, 0, 0);
    f32x4 tB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, awq_operand(wb[0]), zero4, 0, 0, 0);
    f32x4 xsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, ones, zero4, 0, 0, 0);
    tA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, awq_operand(wa[1]), tA, 0, 0, 0);
    tB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, awq_operand(wb[1]), tB, 0, 0, 0);
    xsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, ones, xsum, 0, 0, 0);
    // sum_k x (q - z) s = s sum_k x (128 + q) - s (128 + z) sum_k x.  D row
    // kq * 4 + j sits in register j, so with MT = 2 only registers 0 and 1
    // carry rows of X (in lanes kq == 0); the others are never stored.
#pragma unroll
    for (int j = 0; j < (MT < 4 ? MT : 4); ++j) {
      accA[j] = __builtin_fmaf(tA[j], pa.x, accA[j]);
      accB[j] = __builtin_fmaf(tB[j], pb.x, accB[j]);
      accA[j] = __builtin_fmaf(xsum[j], pa.y, accA[j]);
      accB[j] = __builtin_fmaf(xsum[j], pb.y, accB[j]);
    }
  };

  // move a step's codes and X into this wave's LDS rows (the wave's own
  // LDS accesses execute in order, so the previous step's reads are done)
  auto stage = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(u32x4*)(ws + (8 * j + (lane >> 3)) * kAwqRowPitch + q8 * 16) = wr[slot][j];
#pragma unroll
    for (int v = 0; v < XV; ++v)
      *(u32x4*)(xs + (2 * v + (lane >> 5)) * kAwqXPitch + (lane & 31) * 16) = awq_x_order(xr[slot][v]);
  };

  if (nsteps > 0) {
    int s0 = 0;
    // steady state: whole steps only, every slot refilled right after use
    for (; s0 + 2 * D <= nsteps; s0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        stage(d);
        issue(d, s0 + D + d);
        const int gs = g0 + (s0 + d) * kAwqStepG;
#pragma unroll
        for (int i = 0; i < kAwqStepG; ++i) group(gs + i, i);
      }
    }
    // tail: fewer than 2 D steps left, the first D of them in flight
#pragma unroll
    for (int d = 0; d < 2 * D; ++d) {
      const int step = s0 + d;
      if (step < nsteps) {
        stage(d % D);
        if (d < D && step + D < nsteps) issue(d, step + D);
        const int gs = g0 + step * kAwqStepG;
#pragma unroll
        for (int i = 0; i < kAwqStepG; ++i)
          if (gs + i < g1) group(gs + i, i);
      }
    }
  }

  // ---- sum the K-range partials in a fixed order, add bias, store -----------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    part[wave][kq * 4 + j][c] = accA[j];
    part[wave][kq * 4 + j][16 + c] = accB[j];
  }
  __syncthreads();
  const uint16_t* bias = (const uint16_t*)args.bias;
  uint16_t* out = (uint16_t*)args.out;
  for (int o = tid; o < 16 * 32; o += 256) {
    const int m = o >> 5, cc = o & 31;
    if (m < rows) {
      float v = part[0][m][cc];
#pragma unroll
      for (int w = 1; w < kAwqWaves; ++w) v += part[w][m][cc];
      if (bias) v += bf16_bits_to_f32(bias[n0 + cc]);
      out[(size_t)(m0 + m) * N + n0 + cc] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

template <int MT, int D>
static hipError_t launch_awq_mt(const AwqArgs& a, hipStream_t stream) {
  const int G = (int)(a.K / 64);
  const size_t lds = (size_t)32 * (G + 2) * 8 + (size_t)kAwqWaves * (32 * kAwqRowPitch + MT * kAwqXPitch);
  dim3 grid((unsigned)(a.N / 32), (unsigned)((a.M + MT - 1) / MT));
  if (G <= 64)
    hipLaunchKernelGGL((awq_w4a16_kernel<MT, D, false>), grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL((awq_w4a16_kernel<MT, D, true>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

// ---- one token: a VALU GEMV ----------------------------------------------------
// M = 1 and K a multiple of 1024 (P = K / 1024): the matrix instructions would
// be mostly padding, and the LDS staging they need lengthens every step's
// latency.  Each wave owns R weight rows (R even):
// * the rows come in pairs, 2 K/2 = 1024 P contiguous bytes; instruction i
//   of a pair reads its bytes 1024 i .. 1024 i + 1023, 16 per lane (fully
//   coalesced), so lane l holds 32 codes -- half a group -- of row
//   (1024 i + 16 l) / (K/2) of the pair, the same k for every pair;
// * all of the wave's codes are requested before any arithmetic (R * 512 P
//   bytes in flight per wave), behind x and the scales;
// * the workgroup stages x once in LDS, in the operand pair order; each lane
//   reads the k it holds per use, and sums it once per piece (sum_k x, for
//   the zero-point term);
// * the R rows' scales and zero-points (contiguous) arrive as two 8-byte
//   loads per lane and are interleaved into a wave-private LDS table of
//   (s, z) pairs;
// * codes become bf16 128 + q (awq_operand) and v_dot2_f32_bf16 accumulates
//   sum_k x (128 + q) in fp32 per piece; acc += s dot - s (128 + z) sum_k x;
// * the R per-lane partials are reduced over the 64 lanes with a butterfly
//   (every exchange halves the rows a lane keeps), fixed order.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

template <int R, int P>
__global__ __launch_bounds__(256) void awq_gemv1_kernel(AwqArgs args) {
  static_assert(R % 2 == 0 && R * 16 * P / 4 <= 64, "row pairs; one 8-byte scale load per lane and table");
  constexpr int K2 = 512 * P, G = 16 * P;
  __shared__ __attribute__((aligned(16))) uint16_t xsh[1024 * P];  // x [K] bf16
  __shared__ uint32_t sz[4][R * G];                                // per wave: (s, z) per row and group
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int N = (int)args.N;
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const uint8_t* codes = (const uint8_t*)args.w_codes;

  // x: 16-byte pieces 256 t + tid of the workgroup
  constexpr int kXPieces = (2 * 1024 * P / 16 + 255) / 256;
  u32x4 xv[kXPieces];
#pragma unroll
  for (int t = 0; t < kXPieces; ++t) {
    const int q = min(256 * t + tid, 2 * 1024 * P / 16 - 1);
    xv[t] = *(const u32x4*)((const uint16_t*)args.x + 8 * q);
  }
  // the R rows' scales and zero-points: lane l loads 4 of each
  constexpr int kSzLanes = R * G / 4;
  const int nvals = (min(row0 + R, N) - row0) * G;  // values that exist
  const int sl = min(lane, kSzLanes - 1);
  u32x2 s4 = {0u, 0u}, z4 = {0u, 0u};
  if (4 * sl < nvals) {
    s4 = *(const u32x2*)((const uint16_t*)args.scales + (size_t)row0 * G + 4 * sl);
    z4 = *(const u32x2*)((const uint16_t*)args.zeros + (size_t)row0 * G + 4 * sl);
  }
  // the codes, all pairs at once
  u32x4 w[R / 2][P];
#pragma unroll
  for (int p = 0; p < R / 2; ++p) {
    const int pr = min(row0 + 2 * p, N - 2);
#pragma unroll
    for (int i = 0; i < P; ++i)
      w[p][i] = __builtin_nontemporal_load((const u32x4*)(codes + (size_t)pr * K2 + 1024 * i + 16 * lane));
  }
  // every load above is issued before any arithmetic (the scheduler would
  // otherwise interleave them and keep only a few in flight)
  __builtin_amdgcn_sched_barrier(0);

  // x in LDS, each 8 values in operand order
#pragma unroll
  for (int t = 0; t < kXPieces; ++t)
    if (256 * t + tid < 2 * 1024 * P / 16) *(u32x4*)(xsh + 8 * (256 * t + tid)) = awq_x_order(xv[t]);
  if (lane < kSzLanes) {
    u32x4 v;
    v[0] = __builtin_amdgcn_perm(z4[0], s4[0], 0x05040100u);  // (s, z) of value 4 lane
    v[1] = __builtin_amdgcn_perm(z4[0], s4[0], 0x07060302u);
    v[2] = __builtin_amdgcn_perm(z4[1], s4[1], 0x05040100u);
    v[3] = __builtin_amdgcn_perm(z4[1], s4[1], 0x07060302u);
    *(u32x4*)&sz[wave][4 * lane] = v;
  }
  lds_barrier();

  // the lane's pieces: byte b_i of row r_i of each pair, codes k = 2 b_i ..
  // 2 b_i + 31 (group b_i / 32), and sum_k x over them
  float xs[P];
  int prow[P], pb[P];
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int o = 1024 * i + 16 * lane;
    prow[i] = o >= K2 ? 1 : 0;
    pb[i] = o - prow[i] * K2;
    float t = 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 xq = *(const u32x4*)(xsh + 2 * pb[i] + 8 * h);
#pragma unroll
      for (int d = 0; d < 4; ++d) t = dot2_bf16(xq[d], kOnes, t);
    }
    xs[i] = t;
  }
  float part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) part[r] = 0.f;
#pragma unroll
  for (int p = 0; p < R / 2; ++p) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      float d = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const u32x4 xq = *(const u32x4*)(xsh + 2 * pb[i] + 8 * h);
        const u32x4 op = __builtin_bit_cast(u32x4, awq_operand(w[p][i][h]));
#pragma unroll
        for (int e = 0; e < 4; ++e) d = dot2_bf16(op[e], xq[e], d);
      }
      const int r = 2 * p + prow[i];
      const uint32_t sp = sz[wave][r * G + (pb[i] >> 5)];
      const float s = bf16_lo(sp);
      const float cz = -s * (128.0f + bf16_hi(sp));  // exact
      // the lane's two rows of the pair get their pieces in a fixed order
      const float add = __fmaf_rn(cz, xs[i], s * d);
      if (prow[i]) part[2 * p + 1] += add;
      else part[2 * p] += add;
    }
  }
  // butterfly over the lanes: after it lane l holds the sum of row
  // l >> (6 - log2 R)
  int bit = 32;
#pragma unroll
  for (int n = R; n > 1; n >>= 1, bit >>= 1) {
    const bool up = (lane & bit) != 0;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
      const float send = up ? part[j] : part[n / 2 + j];
      const float keep = up ? part[n / 2 + j] : part[j];
      part[j] = keep + __shfl_xor(send, bit, 64);
    }
  }
  for (; bit >= 1; bit >>= 1) part[0] += __shfl_xor(part[0], bit, 64);
  const int per = 64 / R;
  const int row = row0 + lane / per;
  if (lane % per == 0 && row < N) {
    const float bv = args.bias ? bf16_bits_to_f32(((const uint16_t*)args.bias)[row]) : 0.f;
    ((uint16_t*)args.out)[row] = (uint16_t)f32_to_bf16_bits(part[0] + bv);
  }
}

template <int R, int P>
static hipError_t launch_awq_gemv1(const AwqArgs& a, hipStream_t stream) {
  const unsigned blocks = (unsigned)((a.N + 4 * R - 1) / (4 * R));
  hipLaunchKernelGGL((awq_gemv1_kernel<R, P>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// weight rows per wave of the one-token kernel (4 measured fastest of 2..16)
constexpr int kAwqGemvRows = 4;

hipError_t launch_awq_gemv(const AwqArgs& a, hipStream_t stream) {
  if (a.M == 1 && a.K % 1024 == 0 && a.K <= 4096) {
    switch (a.K / 1024) {
      case 1: return launch_awq_gemv1<kAwqGemvRows, 1>(a, stream);
      case 2: return launch_awq_gemv1<kAwqGemvRows, 2>(a, stream);
      case 3: return launch_awq_gemv1<kAwqGemvRows, 3>(a, stream);
      default: return launch_awq_gemv1<kAwqGemvRows, 4>(a, stream);
    }
  }
  if (a.M <= 2) return launch_awq_mt<2, 1>(a, stream);
  if (a.M <= 4) return launch_awq_mt<4, 1>(a, stream);
  return launch_awq_mt<16, 1>(a, stream);
}

}  // namespace svdq
