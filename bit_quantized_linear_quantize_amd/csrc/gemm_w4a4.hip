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
// of 32 x 32; 64 columns of K per stage, v_mfma_f32_32x32x16_f16.  A goes
// from memory straight into a ring of three LDS stage buffers
// (buffer_load ... lds, rows of 128 bytes with XOR-swizzled 16-byte chunks:
// conflict-free operand reads), issued three stages ahead.  W codes and
// scales are loaded two stages ahead into registers, converted, and written
// to one of two padded LDS stage buffers among the matrix instructions of the
// previous stage.  Tiles are visited in groups of 4 M-tiles, mapped so that
// the workgroups on one XCD share A and W tiles in its L2.
// Low-rank up: lora_act (fp32) split into bf16 hi + lo, times lora_up, with
// bf16 matrix instructions accumulating into the same registers.
//
// PARTIALS=true is the parity export: the same staging and matrix
// instructions with unit scales (A from packed codes), writing the exact
// per-group integer partials (nvfp4: doubled E2M1 codes) instead.

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace svdq {

constexpr int kBM = 256;
constexpr int kBN = 192;
constexpr int kBK = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWM = 4;                    // waves along M
constexpr int kIB = kBM / (32 * kWM);     // 32-row blocks per wave (2)
constexpr int kJB = kBN / (32 * (kWaves / kWM));  // 32-column blocks per wave (3)
constexpr int kRP = kThreads / 8;         // tile rows per register-loader pass (8 threads per row)
constexpr int kAP = kBM / kRP;            // parity export: A pieces per thread and stage (4)
constexpr int kWP = kBN / kRP;            // W pieces per thread and stage (3)
constexpr int kGroupM = 4;
constexpr int kAStages = 3;               // A ring depth
constexpr int kARow = 128;                // A LDS row: 64 fp16 in 8 XOR-swizzled 16-byte chunks
constexpr int kWRow = 144;                // W LDS row: 64 fp16 + 16 pad
constexpr int kADma = kBM * 8 / kThreads; // A direct-to-LDS loads per thread and stage (4)
static_assert(kAP % 4 == 0 && kWP == 3 && kThreads >= kBN && kADma * kThreads == kBM * 8, "loader layout");

template <int I>
using IC = std::integral_constant<int, I>;

// Epilogues: plain bias + bf16 store; the MLP fusion (GELU and nvfp4
// quantization for the next layer); the QKV fusion (RMSNorm and RoPE).
constexpr int kEpiStore = 0;
constexpr int kEpiGelu = 1;
constexpr int kEpiQk = 2;
constexpr int kEpiSplit = 3;  // split K: fp32 partials

// QKV fusion column order.  The output is q | k | v with heads of 128
// columns; a 192-column tile cannot hold whole heads of q or k in the natural
// order, so column tile t of the 2 H tiles takes the 128 columns of head t
// of q | k and 64 columns of v (two tiles' v columns make one head), and
// RMSNorm needs no data from another workgroup.
constexpr int kHeadDim = 128;
static_assert(2 * (kBN - kHeadDim) == kHeadDim, "the v columns of two tiles make one head");
__device__ __forceinline__ int qk_col(int nt, int c, int qk_cols) {
  return c < kHeadDim ? nt * kHeadDim + c : qk_cols + nt * (kBN - kHeadDim) + (c - kHeadDim);
}

// Workgroup barrier for the main loop: this wave's LDS reads and writes are
// complete (lgkmcnt 0), and the compiler moves no memory access across it.
// Unlike a release fence it does not wait for the wave's direct-to-LDS loads
// that are still in flight for later stages.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Position of 16-byte chunk c (columns 8c .. 8c+7 of the stage) in A row
// `row`: the XOR spreads the 16 rows one matrix-instruction operand read
// covers over all 64 banks.
__device__ __forceinline__ int a_pos(int row, int c) { return c ^ ((row >> 1) & 7); }

// One stage of raw W (and, for the parity export, A) data in registers.  Every
// thread has the same role: W piece j = 4 bytes of codes for columns 8c ..
// 8c+7 (c = tid % 8) of tile row tid/8 + 64 j, and its scale; A piece i
// likewise for A row tid/8 + 64 i.
struct RawStage {
  uint32_t w[kWP];
  // the scale of each W piece, kept in its loaded width (a widening right
  // after the load would make the wave wait for the load there)
  uint8_t sw8[kWP];    // nvfp4: E4M3 byte
  uint16_t sw16[kWP];  // int4: bf16 bits
  uint32_t a[kAP];     // parity export only
};

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

// MLP fusion epilogue: wave-private LDS tile of GELU outputs, 64 rows x 96
// bf16 columns, rows padded to 208 bytes (conflict-free row-wise and
// operand-layout reads).
constexpr int kGeluRow = 208;

// GELU with the exact erf of every bf16 value, rounded to bf16 (the table is
// generated at build time in double precision: gelu_bf16_gen.py).  The epilogue's
// GELU input is a bf16 value, so one lookup gives the correctly rounded result.
#include "gelu_bf16_table.inc"

// The MLP fusion epilogue of one wave ("Fused kernels" of the Nunchaku Lite
// docs page: the MLP's GELU and the quantization for the down projection in
// the up projection's epilogue).  acc holds this wave's 64 x 96 block of the
// up projection before its bias.  Steps:
//  1. g = bf16(GELU(bf16(acc + bias))) -- the values a bf16 up output followed
//     by a bf16 GELU would give; GELU by the table kGeluBf16 -- into the
//     wave's LDS tile `tile_base` (+ 64 kGeluRow for odd waves);
//  2. the next layer's low-rank activations: x = fl32(g * (1 / smooth_next))
//     in the 16x16x32 bf16 operand layout, split hi + lo, times
//     next_lora_down, added into next_lora_act with fp32 atomics (one
//     partial per wave and tile);
//  3. lane l takes tile row l: the same x, nvfp4 per 16 columns
//     (nvfp4_quant16, the quantize kernel's reading); the next layer's
//     product operand e2m1 * dec(s8) as fp16 overwrites the lane's own tile
//     row, and the wave then stores the tile with consecutive lanes on
//     consecutive 16-byte pieces of a row.
// Columns past N have 1/smooth 0 (x = 0) and are not stored; rows past M are
// not stored.
__device__ __forceinline__ void gelu_quant_epilogue(const GemmArgs& args, f32x16 (&acc)[kIB][kJB], int m0, int n0,
                                                    int wave, int wm, int wn, int lane, int l32, int h,
                                                    const float* nmu, uint8_t* tile_base) {
  const int M = (int)args.M, N = (int)args.N;
  uint8_t* gt = tile_base + (wave & 1) * (64 * kGeluRow);
  // every wave has left the main loop (its LDS reads are done) and every
  // direct-to-LDS load has landed before the buffers are reused
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // 1. the GELU tile
  const uint16_t* bias = (const uint16_t*)args.bias;
#pragma unroll
  for (int j = 0; j < kJB; ++j) {
    const int col = n0 + wn * (kJB * 32) + j * 32 + l32;
    const float bv = (bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        *(uint16_t*)(gt + r * kGeluRow + (j * 32 + l32) * 2) = kGeluBf16[f32_to_bf16_bits(acc[i][j][e] + bv)];
      }
  }
  // (the wave's own LDS writes and reads execute in order)

  // 2 and 3 both read the next layer's 1 / smooth of this wave's columns
  const float* mu = nmu + wn * (kJB * 32);
  // 2. the next layer's low-rank down projection of this tile's columns (it
  // reads the GELU values before step 3 replaces them)
  const int nrank = args.next_rank;
  if (nrank > 0) {
    const int r16 = lane & 15, q = lane >> 4;
    bf16x8 ahi[4][3], alo[4][3];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const f32x4 mu0 = *(const f32x4*)(mu + ks * 32 + 8 * q);
      const f32x4 mu1 = *(const f32x4*)(mu + ks * 32 + 8 * q + 4);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const u32x4 g = *(const u32x4*)(gt + (rb * 16 + r16) * kGeluRow + (ks * 32 + 8 * q) * 2);
        u32x4 hi4, lo4;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float a = __fmul_rn(bf16_lo(g[p]), p < 2 ? mu0[2 * p] : mu1[2 * p - 4]);
          const float b = __fmul_rn(bf16_hi(g[p]), p < 2 ? mu0[2 * p + 1] : mu1[2 * p - 3]);
          const uint32_t hh = bf16x2_rne(a, b);
          hi4[p] = hh;
          lo4[p] = bf16x2_rne(__fsub_rn(a, bf16_lo(hh)), __fsub_rn(b, bf16_hi(hh)));
        }
        ahi[rb][ks] = __builtin_bit_cast(bf16x8, hi4);
        alo[rb][ks] = __builtin_bit_cast(bf16x8, lo4);
      }
    }
    // next_lora_down [nrank, N]: reads past the end of the array return zero
    const __amdgpu_buffer_rsrc_t ld_rs = make_rsrc(args.next_lora_down, (size_t)nrank * N * 2);
    for (int rk = 0; rk < nrank; rk += 16) {
      bf16x8 b[3];
#pragma unroll
      for (int ks = 0; ks < 3; ++ks)
        b[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               ld_rs, ((rk + r16) * N + n0 + wn * (kJB * 32) + ks * 32 + 8 * q) * 2,
                                               0, 0));
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[rb][ks], b[ks], d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[rb][ks], b[ks], d, 0, 0, 0);
        }
        // D: lane (c, q) holds rows 4q + j of the row block, rank column c
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + wm * 64 + rb * 16 + 4 * q + j;
          if (m < M) unsafeAtomicAdd(args.next_lora_act + (size_t)m * nrank + rk + r16, d[j]);
        }
      }
    }
  }

  // 3. quantization for the next layer, one tile row per lane; each group's
  // fp16 operand replaces its GELU values in the lane's own tile row, then
  // the wave copies the tile out with row-contiguous lanes
  {
    uint8_t* rowp = gt + lane * kGeluRow;
#pragma unroll
    for (int t = 0; t < 6; ++t) {
      const u32x4 g0 = *(const u32x4*)(rowp + 32 * t);
      const u32x4 g1 = *(const u32x4*)(rowp + 32 * t + 16);
      float x[16];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        x[2 * p] = __fmul_rn(bf16_lo(g0[p]), mu[16 * t + 2 * p]);
        x[2 * p + 1] = __fmul_rn(bf16_hi(g0[p]), mu[16 * t + 2 * p + 1]);
        x[8 + 2 * p] = __fmul_rn(bf16_lo(g1[p]), mu[16 * t + 8 + 2 * p]);
        x[8 + 2 * p + 1] = __fmul_rn(bf16_hi(g1[p]), mu[16 * t + 8 + 2 * p + 1]);
      }
      uint32_t cw0, cw1;
      float S;
      nvfp4_quant16(x, cw0, cw1, S);
      // e2m1 * dec(s8) is an exact fp16 (|v| <= 2688, >= 2^-10)
      const _Float16 S16 = (_Float16)S;
      *(f16x8*)(rowp + 32 * t) = e2m1x8_to_f16_scaled(cw0, S16);
      *(f16x8*)(rowp + 32 * t + 16) = e2m1x8_to_f16_scaled(cw1, S16);
    }
    // copy-out: 16-byte chunk c of the 64 x 192-byte tile, c = 64 i + lane,
    // is row c / 12, bytes 16 (c % 12) of it
    const int c0 = n0 + wn * (kJB * 32);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      const int c = 64 * i + lane;
      const int r = c / 12, k = c - 12 * r;
      const u32x4 v = *(const u32x4*)(gt + r * kGeluRow + 16 * k);
      const int m = m0 + wm * 64 + r;
      if (m < M && c0 + 8 * k < N) *(u32x4*)((_Float16*)args.next_act + (size_t)m * N + c0 + 8 * k) = v;
    }
  }
}

// The QKV fusion epilogue of one wave ("Fused kernels" of the Nunchaku Lite
// docs page: the Q, K and V projections merged with RMSNorm and RoPE).  acc
// holds this wave's 64 x 96 block before the bias; tile columns 0..127 are
// head nt of q | k (q for nt < heads), 128..191 v columns (qk_col).  Wave
// column group wn = 0 holds head dims 0..95, wn = 1 head dims 96..127 and
// the 64 v columns.  Steps:
//  1. h = bf16(acc + bias) into the wave's LDS tile (rows of kGeluRow bytes);
//  2. lane l takes tile row l: the sum of squares of its head columns; the
//     two waves of a row block add theirs through LDS (`ssq`, in a fixed
//     order) and r = 1 / sqrt(sum / 128 + eps);
//  3. each head pair (2i, 2i+1): n = bf16(fl32(fl32(h r) w_d)), then
//     (n_a cos - n_b sin, n_a sin + n_b cos) in fp32, rounded to bf16 in
//     place; v columns keep h;
//  4. the wave stores the tile with consecutive lanes on consecutive 16-byte
//     pieces of a row.
__device__ __forceinline__ void qk_norm_rope_epilogue(const GemmArgs& args, f32x16 (&acc)[kIB][kJB], int m0, int nt,
                                                      int wave, int wm, int wn, int lane, int l32, int h,
                                                      uint8_t* tile_base, float* ssq) {
  const int M = (int)args.M, N = (int)args.N;
  const int heads = args.heads;
  const int qk_cols = 2 * heads * kHeadDim;
  uint8_t* gt = tile_base + (wave & 1) * (64 * kGeluRow);
  // every wave has left the main loop and every direct-to-LDS load has landed
  // before the stage buffers are reused
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // 1. the bf16 projection
  const uint16_t* bias = (const uint16_t*)args.bias;
#pragma unroll
  for (int j = 0; j < kJB; ++j) {
    const int col = qk_col(nt, wn * (kJB * 32) + j * 32 + l32, qk_cols);
    const float bv = bias ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        *(uint16_t*)(gt + r * kGeluRow + (j * 32 + l32) * 2) = (uint16_t)f32_to_bf16_bits(acc[i][j][e] + bv);
      }
  }
  // (the wave's own LDS writes and reads execute in order)

  // 2. RMSNorm factor of the lane's row
  uint8_t* rowp = gt + lane * kGeluRow;
  const int nhead = wn == 0 ? kJB * 32 : kHeadDim - kJB * 32;  // head columns of this wave (96 | 32)
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < 12; ++t) {
    if (8 * t < nhead) {
      const u32x4 v = *(const u32x4*)(rowp + 16 * t);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = bf16_lo(v[p]), b = bf16_hi(v[p]);
        ss = __fmaf_rn(a, a, ss);
        ss = __fmaf_rn(b, b, ss);
      }
    }
  }
  const int trow = wm * 64 + lane;  // row of the workgroup tile
  ssq[wn * kBM + trow] = ss;
  lds_barrier();
  const float tot = __fadd_rn(ssq[trow], ssq[kBM + trow]);
  const float rr = __fdiv_rn(1.0f, __fsqrt_rn(__fmaf_rn(tot, 1.0f / kHeadDim, args.eps)));

  // 3. normalize and rotate the head columns in place
  const uint32_t* nw = (const uint32_t*)(nt < heads ? args.q_norm : args.k_norm);  // bf16 pairs
  const int m = m0 + trow;
  const size_t trow_off = (size_t)min(m, M - 1) * (kHeadDim / 2);
  const float* cs = args.rope_cos + trow_off;
  const float* sn = args.rope_sin + trow_off;
  const int d0 = wn * (kJB * 32);  // head dim of the wave's first column
#pragma unroll
  for (int t = 0; t < 12; ++t) {
    if (8 * t < nhead) {
      const u32x4 v = *(const u32x4*)(rowp + 16 * t);
      const int pr = (d0 + 8 * t) >> 1;  // first pair of the piece
      const f32x4 c4 = *(const f32x4*)(cs + pr);
      const f32x4 s4 = *(const f32x4*)(sn + pr);
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t wp = nw[pr + p];
        const float na = __uint_as_float(f32_to_bf16_bits(__fmul_rn(__fmul_rn(bf16_lo(v[p]), rr), bf16_lo(wp))) << 16);
        const float nb = __uint_as_float(f32_to_bf16_bits(__fmul_rn(__fmul_rn(bf16_hi(v[p]), rr), bf16_hi(wp))) << 16);
        const float oa = __fsub_rn(__fmul_rn(na, c4[p]), __fmul_rn(nb, s4[p]));
        const float ob = __fadd_rn(__fmul_rn(na, s4[p]), __fmul_rn(nb, c4[p]));
        o[p] = bf16x2_rne(oa, ob);
      }
      *(u32x4*)(rowp + 16 * t) = o;
    }
  }

  // 4. copy-out: 16-byte chunk c of the 64 x 192-byte tile, c = 64 i + lane,
  // is row c / 12, bytes 16 (c % 12) of it; a piece never crosses a head edge
  uint16_t* out = (uint16_t*)args.out;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const int c = 64 * i + lane;
    const int r = c / 12, k = c - 12 * r;
    const u32x4 v = *(const u32x4*)(gt + r * kGeluRow + 16 * k);
    const int mr = m0 + wm * 64 + r;
    const int col = qk_col(nt, wn * (kJB * 32) + 8 * k, qk_cols);
    if (mr < M) *(u32x4*)(out + (size_t)mr * N + col) = v;
  }
}

template <int PREC, int RB, bool PARTIALS, int EPI = kEpiStore>
__global__ __launch_bounds__(kThreads) void gemm_w4a4_lora_up_kernel(GemmArgs args) {
  // separate LDS objects, selected at compile time, so that the compiler can
  // tell the buffers apart from those that direct-to-LDS loads are filling
  __shared__ __attribute__((aligned(16))) uint8_t lds_a0[kBM * kARow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a1[kBM * kARow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a2[kBM * kARow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_w0[kBN * kWRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_w1[kBN * kWRow];
  __shared__ float wexp[kBN];   // int4: 2^F[n] of this tile's weight rows
  __shared__ float wdown[kBN];  // int4: 2^-F[n]
  __shared__ float nmu[kBN];    // MLP fusion: 1 / smooth of the next layer for this tile's columns
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kWM, wn = wave / kWM;
  const int M = (int)args.M, K = (int)args.K, N = (int)args.N;
  const int K2 = K >> 1;
  const int nmt = (M + kBM - 1) / kBM, nnt = (N + kBN - 1) / kBN;
  int mt, nt;
  tile_of(blockIdx.x, nmt, nnt, mt, nt);
  const int m0 = mt * kBM, n0 = nt * kBN;
  // split K: this workgroup's stages [s0, s0 + nstages) (the loads below take
  // their stage offsets from descriptor bases moved to stage s0)
  constexpr bool kSplit = EPI == kEpiSplit;
  int s0 = 0, nstages = K / kBK;
  if constexpr (kSplit) {
    const int per = (nstages + args.ksplit - 1) / args.ksplit;
    s0 = blockIdx.y * per;
    nstages = min(per, nstages - s0);
  }
  // physical column of tile column c (the QKV fusion reorders columns)
  constexpr bool kQk = EPI == kEpiQk;
  const int qk_cols = kQk ? 2 * args.heads * kHeadDim : 0;
  auto pcol = [&](int c) -> int {
    if constexpr (kQk) return qk_col(nt, c, qk_cols);
    else return n0 + c;
  };
  if constexpr (EPI == kEpiGelu) {
    // read before the first use by the main loop's barriers
    if (tid < kBN) {
      const int col = n0 + tid;
      nmu[tid] = col < N ? __fdiv_rn(1.0f, bf16_bits_to_f32(((const uint16_t*)args.next_smooth)[col])) : 0.f;
    }
  }
  constexpr bool kRowExp = PREC == kInt4 && !PARTIALS;

  // ---- loaders ---------------------------------------------------------------
  // Buffer loads: one descriptor per operand based at this tile's first row,
  // 32-bit lane offsets, the stage offset in a scalar register.  Rows past
  // the end of the matrix, and stages past the last, lie beyond the
  // descriptor's size or in rows that are never used, and read as zero.
  const int lc = tid & 7;    // column chunk: columns 8 lc .. 8 lc + 7 of the stage
  const int lr = tid >> 3;   // tile row of piece 0 (piece i: lr + 64 i)
  const size_t a_row_bytes = PARTIALS ? (size_t)K2 : (size_t)K * 2;
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc((const uint8_t*)args.act + (size_t)m0 * a_row_bytes + s0 * 128,
                                                (size_t)(M - m0) * a_row_bytes - s0 * 128);
  // (the QKV fusion addresses W rows from the matrix start: its tile rows
  // are not contiguous)
  const int w_base = kQk ? 0 : n0;
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc((const uint8_t*)args.w_codes + (size_t)w_base * K2 + s0 * 32,
                                                (size_t)(N - w_base) * K2 - s0 * 32);
  const size_t ws_row_bytes = PREC == kInt4 ? (size_t)(K >> 6) * 2 : (size_t)(K >> 4);
  const int ws_s0 = s0 * (PREC == kInt4 ? 2 : 4);  // scale bytes per stage and row
  const __amdgpu_buffer_rsrc_t ws_rs = make_rsrc((const uint8_t*)args.w_scales + (size_t)w_base * ws_row_bytes + ws_s0,
                                                 PARTIALS ? 0 : (size_t)(N - w_base) * ws_row_bytes - ws_s0);
  // stages past the last read through an empty descriptor: all zeros
  const __amdgpu_buffer_rsrc_t zero_rs = make_rsrc(args.w_codes, 0);
  int w_off[kWP], ws_off[kWP], pa_off[kAP];
#pragma unroll
  for (int j = 0; j < kWP; ++j) {
    const int wrow = kQk ? pcol(lr + kRP * j) : lr + kRP * j;  // row from the descriptor base
    w_off[j] = wrow * K2 + lc * 4;
    ws_off[j] = wrow * (int)ws_row_bytes + (PREC == kNvfp4 ? (lc >> 1) : 0);
  }
#pragma unroll
  for (int i = 0; i < kAP; ++i) pa_off[i] = (lr + kRP * i) * K2 + lc * 4;
  // A (fp16) goes straight from memory to LDS: load d of a wave fills the
  // 1 KB of LDS units u0 .. u0+63 (u0 = 64 (kADma wave + d)), lane l unit
  // u0 + l = row u/8, position u%8, which holds chunk a_pos(row, u%8).
  int dma_off[kADma];
#pragma unroll
  for (int d = 0; d < kADma; ++d) {
    const int u = (wave * kADma + d) * 64 + lane;
    const int row = u >> 3;
    dma_off[d] = row * (int)a_row_bytes + a_pos(row, u & 7) * 16;
  }

  auto abuf = [&](auto c) -> uint8_t* {
    constexpr int i = decltype(c)::value % kAStages;
    if constexpr (i == 0) return lds_a0;
    else if constexpr (i == 1) return lds_a1;
    else return lds_a2;
  };
  auto wbuf = [&](auto c) -> uint8_t* {
    if constexpr (decltype(c)::value % 2 == 0) return lds_w0;
    else return lds_w1;
  };

  // loads of stage s: A into A buffer ab (direct to LDS), W into r
  auto group = [&](RawStage& r, int s, auto ab) {
    const bool live = s < nstages;
    const __amdgpu_buffer_rsrc_t ars = live ? a_rs : zero_rs;
    const __amdgpu_buffer_rsrc_t wrs = live ? w_rs : zero_rs;
    const __amdgpu_buffer_rsrc_t srs = live ? ws_rs : zero_rs;
    if constexpr (!PARTIALS) {
      uint8_t* dst = abuf(ab) + wave * (kADma * 64 * 16);
#pragma unroll
      for (int d = 0; d < kADma; ++d)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (__attribute__((address_space(3))) void*)(dst + d * 1024), 16,
                                                 dma_off[d], s * 128, 0, 0);
      // the W loads of the stage stay behind its A loads: a wave that has
      // waited for its W registers has also received its A stage
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < kWP; ++j) {
      r.w[j] = __builtin_amdgcn_raw_buffer_load_b32(wrs, w_off[j], s * 32, 0);
      if constexpr (PREC == kNvfp4 && !PARTIALS) r.sw8[j] = __builtin_amdgcn_raw_buffer_load_b8(srs, ws_off[j], s * 4, 0);
      if constexpr (PREC == kInt4 && !PARTIALS) r.sw16[j] = __builtin_amdgcn_raw_buffer_load_b16(srs, ws_off[j], s * 2, 0);
    }
    if constexpr (PARTIALS) {
#pragma unroll
      for (int i = 0; i < kAP; ++i) r.a[i] = __builtin_amdgcn_raw_buffer_load_b32(ars, pa_off[i], s * 32, 0);
    }
  };

  const int G64 = K >> 6;
  float wdn[kWP];  // int4: 2^-F[n] of this thread's weight rows (set after the prologue)

  // staging of one raw stage in three parts (part p: W piece p and, for the
  // parity export, A pieces of part p), so that it can be interleaved with
  // the matrix instructions of the previous stage
  auto store_part = [&](uint8_t* Ta, uint8_t* Tw, const RawStage& r, int p) {
    if constexpr (PARTIALS) {
      // unit scales; nvfp4 doubles the E2M1 codes so that they are integers
      const _Float16 one = (_Float16)(PREC == kInt4 ? 1.0f : 2.0f);
#pragma unroll
      for (int i = 0; i < kAP; ++i) {
        if (i * 3 / kAP != p) continue;
        const int row = lr + kRP * i;
        *(f16x8*)(Ta + row * kARow + a_pos(row, lc) * 16) =
            PREC == kInt4 ? int4x8_to_f16_scaled(r.a[i], one) : e2m1x8_to_f16_scaled(r.a[i], one);
      }
    }
    const int wrow = lr + kRP * p;
    _Float16 sc = (_Float16)(PREC == kInt4 ? 1.0f : 2.0f);
    if constexpr (!PARTIALS) {
      if constexpr (PREC == kInt4)
        sc = (_Float16)(bf16_bits_to_f32(r.sw16[p]) * wdn[p]);  // exact: a power of two
      else
        sc = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sw8[p], 0);
    }
    *(f16x8*)(Tw + wrow * kWRow + lc * 16) =
        PREC == kInt4 ? int4x8_to_f16_scaled(r.w[p], sc) : e2m1x8_to_f16_scaled(r.w[p], sc);
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

  // operands of two k steps of 16 (set ks & 1); the A offsets of the
  // swizzled rows are fixed per k step
  int a_rd[kIB][4];
#pragma unroll
  for (int i = 0; i < kIB; ++i) {
    const int row = wm * (kIB * 32) + i * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a_rd[i][ks] = row * kARow + a_pos(row, 2 * ks + h) * 16;
  }
  f16x8 aop[2][kIB], bop[2][kJB];
  auto rd = [&](const uint8_t* Ta, const uint8_t* Tw, int ks, int set) {
#pragma unroll
    for (int i = 0; i < kIB; ++i) aop[set][i] = *(const f16x8*)(Ta + a_rd[i][ks]);
#pragma unroll
    for (int j = 0; j < kJB; ++j)
      bop[set][j] = *(const f16x8*)(Tw + (wn * (kJB * 32) + j * 32 + l32) * kWRow + ks * 32 + h * 16);
  };

  // One stage s: 4 k steps of 16, each 6 products.  On entry the operands of
  // k step 0 are in set 0; those of step ks+1 are read before the products of
  // step ks are issued.  The raw stage r (stage s+1) is staged among the
  // products of steps 0..2 (its VALU work and LDS writes issue while the
  // matrix instructions execute).  The barrier comes before the products of
  // the last step: every wave has then finished reading stage s and writing
  // stage s+1 (and holds its own A loads of stage s+1, which precede the W
  // loads it waited for), so the operands of the next stage's step 0 are read
  // while those products execute, and stage s+3 is loaded into the A buffer
  // of stage s and into r.
  // (P = s mod 6 at compile time: A buffer P mod 3, W buffer P mod 2)
  auto compute = [&](auto P, int s, RawStage& r) {
    constexpr int p = decltype(P)::value;
    uint8_t* Ta = abuf(IC<p>{});
    uint8_t* Tw = wbuf(IC<p>{});
    uint8_t* Na = abuf(IC<p + 1>{});
    uint8_t* Nw = wbuf(IC<p + 1>{});
    const bool live = s < nstages;  // (parity export: only live stages have partials)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
        rd(Ta, Tw, ks + 1, (ks + 1) & 1);
      } else {
        stage_barrier();
        rd(Na, Nw, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int j = 0; j < kJB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[ks & 1][i], bop[ks & 1][j], acc[i][j], 0, 0, 0);
      if (ks < 3) store_part(Na, Nw, r, ks);
      if (ks == 3) group(r, s + 3, IC<p>{});
      if constexpr (!PARTIALS) {
        // order: LDS reads of the next operands, then the products
        // interleaved with the staging arithmetic, then the staging write
        __builtin_amdgcn_sched_group_barrier(0x100, kIB + kJB, 0);
        if (ks < 3) {
#pragma unroll
          for (int m = 0; m < kIB * kJB; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
      }
      if constexpr (PARTIALS && PREC == kNvfp4) {
        if (live) partial_store(s * 4 + ks, nstages * 4);
      }
    }
    if constexpr (PARTIALS && PREC == kInt4) {
      if (live) partial_store(s, nstages);
    }
  };

  // ---- main loop -------------------------------------------------------------
  // Loads run three stages ahead for A (a ring of three LDS buffers) and two
  // for W (two raw stages in registers, staged into two LDS buffers).  The
  // loop is unrolled by two so that every register array index is a
  // compile-time constant (a runtime index would move the array to scratch).
  RawStage r0, r1;
  group(r0, 0, IC<0>{});
  group(r1, 1, IC<1>{});
  // int4: per weight row the power of two 2^-F that makes every q * s_w * 2^-F
  // an exact fp16, from the row's largest group scale (its loads overlap the
  // first two stages' loads)
  if constexpr (kRowExp) {
    if (tid < kBN) {
      // the row's scales, two per load (G64 is even: rows are 4-byte aligned)
      const uint16_t* srow = (const uint16_t*)args.w_scales + (size_t)(kQk ? pcol(tid) : min(n0 + tid, N - 1)) * G64;
      float m = 0.f;
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
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kWP; ++j) wdn[j] = wdown[lr + kRP * j];
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) store_part(lds_a0, lds_w0, r0, p);
  group(r0, 2, IC<2>{});
  stage_barrier();  // (each wave has its stage-0 A loads: they precede the W loads it staged)
  rd(lds_a0, lds_w0, 0, 0);
  // Six stages per iteration (the A ring of three times the two raw register
  // stages), all straight-line code.  Stages past the last (up to four when
  // the stage count is not a multiple of six) load zeros and add nothing.
  for (int s = 0; s < nstages; s += 6) {
    compute(IC<0>{}, s, r1);
    compute(IC<1>{}, s + 1, r0);
    compute(IC<2>{}, s + 2, r1);
    compute(IC<3>{}, s + 3, r0);
    compute(IC<4>{}, s + 4, r1);
    compute(IC<5>{}, s + 5, r0);
  }
  // the direct-to-LDS loads of the stages past the end are still in flight
  __builtin_amdgcn_s_waitcnt(0);

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
    // (split K: in split 0 only)
    if constexpr (RB > 0) {
      if (!kSplit || blockIdx.y == 0) {
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
            const int tc = wn * (kJB * 32) + j * 32 + l32;
            const int col = kQk ? pcol(tc) : min(n0 + tc, N - 1);
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
    }
    if constexpr (EPI == kEpiGelu) {
      gelu_quant_epilogue(args, acc, m0, n0, wave, wm, wn, lane, l32, h, nmu,
                          wave < 2 ? lds_a0 : wave < 4 ? lds_a1 : wave < 6 ? lds_a2 : lds_w0);
    } else if constexpr (kQk) {
      qk_norm_rope_epilogue(args, acc, m0, nt, wave, wm, wn, lane, l32, h,
                            wave < 2 ? lds_a0 : wave < 4 ? lds_a1 : wave < 6 ? lds_a2 : lds_w0, (float*)lds_w1);
    } else if constexpr (kSplit) {
      // ---- fp32 partials of this split (no bias) ------------------------------
      float* part = args.partial + (size_t)blockIdx.y * M * N;
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        const int col = n0 + wn * (kJB * 32) + j * 32 + l32;
#pragma unroll
        for (int i = 0; i < kIB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = m0 + wm * (kIB * 32) + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
            if (row < M && col < N) part[(size_t)row * N + col] = acc[i][j][e];
          }
      }
    } else {
      // ---- bias + bf16 store ------------------------------------------------
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
}

template <int PREC, bool PARTIALS, int EPI>
static hipError_t dispatch_rank(const GemmArgs& a, hipStream_t s) {
  const unsigned tiles = (unsigned)(((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN));
  dim3 grid(tiles, EPI == kEpiSplit ? (unsigned)a.ksplit : 1u), block(kThreads);
  if constexpr (PARTIALS) {
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, 0, true, kEpiStore>), grid, block, 0, s, a);
  } else {
#define SVDQ_K2_CASE(rb)                                                                            \
  case rb:                                                                                          \
    hipLaunchKernelGGL((gemm_w4a4_lora_up_kernel<PREC, rb, false, EPI>), grid, block, 0, s, a);   \
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

__global__ __launch_bounds__(256) void gelu_table_copy_kernel(uint16_t* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  out[i] = kGeluBf16[i];
}

// Parity export: the 65536-entry bf16 GELU table.
hipError_t launch_gelu_table_copy(uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(gelu_table_copy_kernel, dim3(256), dim3(256), 0, stream, out);
  return hipGetLastError();
}

// Split K: out[m, n] = bf16(sum_j partial[j, m, n] + bias[n]), the splits
// added in order (deterministic); 8 columns per thread (N % 64 == 0).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int ksplit, int64_t M,
                                                            int64_t N, const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;  // first element
  if (i >= M * N) return;
  const int64_t n = i % N;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  for (int j = 0; j < ksplit; ++j) {
    const f32x4* p = (const f32x4*)(partial + (size_t)j * M * N + i);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[c] += a[c];
      acc[4 + c] += b[c];
    }
  }
  u32x4 o;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float b0 = bias ? bf16_bits_to_f32(bias[n + 2 * c]) : 0.f;
    const float b1 = bias ? bf16_bits_to_f32(bias[n + 2 * c + 1]) : 0.f;
    o[c] = f32_to_bf16_bits(acc[2 * c] + b0) | (f32_to_bf16_bits(acc[2 * c + 1] + b1) << 16);
  }
  *(u32x4*)(out + i) = o;
}

hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N, const void* bias, void* out,
                                hipStream_t stream) {
  const int64_t threads = M * N / 8;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, partial,
                     ksplit, M, N, (const uint16_t*)bias, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream) {
  const bool partials = a.partials != nullptr;
  const int epi = a.next_act != nullptr ? kEpiGelu : a.heads > 0 ? kEpiQk : a.ksplit > 1 ? kEpiSplit : kEpiStore;
  if (a.precision == kInt4) {
    if (partials) return dispatch_rank<kInt4, true, kEpiStore>(a, stream);
    if (epi == kEpiGelu) return dispatch_rank<kInt4, false, kEpiGelu>(a, stream);
    if (epi == kEpiQk) return dispatch_rank<kInt4, false, kEpiQk>(a, stream);
    if (epi == kEpiSplit) return dispatch_rank<kInt4, false, kEpiSplit>(a, stream);
    return dispatch_rank<kInt4, false, kEpiStore>(a, stream);
  }
  if (partials) return dispatch_rank<kNvfp4, true, kEpiStore>(a, stream);
  if (epi == kEpiGelu) return dispatch_rank<kNvfp4, false, kEpiGelu>(a, stream);
  if (epi == kEpiQk) return dispatch_rank<kNvfp4, false, kEpiQk>(a, stream);
  if (epi == kEpiSplit) return dispatch_rank<kNvfp4, false, kEpiSplit>(a, stream);
  return dispatch_rank<kNvfp4, false, kEpiStore>(a, stream);
}

}  // namespace svdq
