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
// Workgroup tile 256 (M) x 192 (N) -- 256 workgroups for a 4096 x 3072
// output, one per CU -- with 8 waves (4 x 2), each wave 64 x 96 = 2 x 3 blocks
// of 32 x 32.  Tiles are visited in groups of 4 M-tiles, mapped so that the
// workgroups on one XCD share A and W tiles in its L2.  Two datapaths:
//
// int4 -- fp8 operands, group scales applied per group.  Every code |q| <= 7
// is an exact fp8 E4M3 value, so one v_mfma_f32_32x32x64_f8f6f4 per 32 x 32
// block and group (K = 64) gives the group's exact integer sums P.  The bf16
// group scales (which the instruction's power-of-two block scales cannot
// express) are applied as acc += P * (s_x s_w), the 32 x 32 scale products
// (exact in fp32) coming from one bf16 outer-product instruction
// (v_mfma_f32_32x32x8_bf16) and the accumulation from one FMA per output.
// The quantize kernel writes A as E4M3 bytes with bf16 group scales; a stage
// is 128 values of K (two groups).  The matrix work is half that of the fp16
// route below, and it runs at a lower power: the fp16 route on int4 data is
// held back by the clock the chip sustains under full matrix load.
//
// nvfp4 -- scales folded into exact fp16 operands.  An E2M1 code times its
// E4M3 block scale needs at most 2 + 4 significant bits, an exact fp16, so
// one fp16 matrix product with fp32 accumulation over all of K gives
// sum_g s_x s_w P_g (the per-16 scales fit no wider instruction): A arrives
// from the quantize kernel as e2m1 * dec(s8) in fp16; W is converted while
// staging (codes via cvt_scalef32_pk_f16_fp4, times dec(s8)); wtscale is
// applied at the end.  64 values of K per stage, v_mfma_f32_32x32x16_f16.
//
// Both: A goes from memory straight into a ring of three LDS stage buffers
// (buffer_load ... lds, rows of 128 bytes with XOR-swizzled 16-byte chunks:
// conflict-free operand reads), issued three stages ahead (int4: its group
// scales likewise).  W codes and scales are loaded two stages ahead into
// registers, converted, and written to one of two padded LDS stage buffers
// among the matrix instructions of the previous stage.
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

// QKV fusion column order.  The output is q | k | v with heads of D = 32, 64
// or 128 consecutive columns; a 192-column tile cannot hold whole heads of q
// or k in the natural order, so column tile t takes the 128 q | k columns
// 128 t .. 128 t + 127 (whole heads: 128 / D of them) and the 64 v columns
// 64 t .. 64 t + 63, and RMSNorm needs no data from another workgroup.
constexpr int kQkCols = 128;  // q | k columns per tile
static_assert(kBN - kQkCols == 64, "64 v columns per tile");
__device__ __forceinline__ int qk_col(int nt, int c, int qk_cols) {
  return c < kQkCols ? nt * kQkCols + c : qk_cols + nt * (kBN - kQkCols) + (c - kQkCols);
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
// likewise for A row tid/8 + 64 i.  (nvfp4 linear: pieces 0 and 1 are instead
// the two halves of one 8-byte load, columns 16c .. 16c+15 (c = tid % 4, one
// scale block) of tile row tid/4; the scales come at even stages only, the
// four of the stage and the four of the next per row in spa (row tid/4) and
// spb (row 128 + tid/8).)
struct RawStage {
  uint32_t w[kWP];
  u32x2 spa, spb;      // nvfp4 linear
  // the scale of each W piece, kept in its loaded width (a widening right
  // after the load would make the wave wait for the load there)
  uint8_t sw8[kWP];    // nvfp4: E4M3 byte
  uint32_t a[kAP];     // parity export only
};

// int4 as fp8: sixteen sign-magnitude codes (nibble i = column i, low nibble
// first) -> sixteen OCP fp8 E4M3 bytes in column order.  |q| <= 7 is exact in
// E4M3: a table of the eight magnitude bytes (v_perm) plus the sign bit; the
// code 0x8 (-0) gives 0x80, fp8 -0.
__device__ __forceinline__ u32x4 int4x16_to_fp8(u32x2 w) {
  constexpr uint32_t kT0 = 0x44403800u;  // E4M3 bytes of 0, 1, 2, 3
  constexpr uint32_t kT1 = 0x4E4C4A48u;  // of 4, 5, 6, 7
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t v = w[k];
    const uint32_t elo = __builtin_amdgcn_perm(kT1, kT0, v & 0x07070707u) | ((v << 4) & 0x80808080u);  // columns 0 2 4 6
    const uint32_t ehi = __builtin_amdgcn_perm(kT1, kT0, (v >> 4) & 0x07070707u) | (v & 0x80808080u);  // 1 3 5 7
    r[2 * k] = __builtin_amdgcn_perm(ehi, elo, 0x05010400u);      // columns 0 1 2 3
    r[2 * k + 1] = __builtin_amdgcn_perm(ehi, elo, 0x07030602u);  // columns 4 5 6 7
  }
  return r;
}

// One stage of raw W data of the int4 fp8 path in registers (192 rows x 64
// bytes in two loads per thread): wa = 16 bytes of codes (columns
// 32 c .. 32 c + 31 of the stage, c = tid % 4) of tile row tid / 4, wb = 8
// bytes (columns 16 c .. 16 c + 15, c = tid % 8) of tile row 128 + tid / 8;
// and (even stages only) the bf16 scales of two stages' groups.
struct RawStage8 {
  u32x4 wa;
  u32x2 wb;
  uint32_t sw;  // the two bf16 group scales of W row srow (24 rows per wave)
                // of this stage (lanes 0-23, 48-63) or of the next (24-47)
};

// The operands of one 16-wide rank slice of the low-rank up projection, as
// loaded: lora_act (fp32) of the wave's two 32-row blocks, lora_up (bf16) of
// its three 32-column blocks.
struct LoraOps {
  f32x4 a[kIB][2];
  u32x4 b[kJB];
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
// the fused MLP's low-rank exchange: rows of 32 sums + 4 pad floats, so that
// the four 16-lane quarters of a wave write distinct banks
constexpr int kXchRow = 36;
static_assert(2 * kWM * 16 * kXchRow * 4 <= kBN * kWRow, "the exchange fits the second W buffer");

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
//  2. the next layer's low-rank activations of this tile's 192 columns: x =
//     fl32(g * (1 / smooth_next)) in the 16x16x32 bf16 operand layout, split
//     hi + lo, times next_lora_down.  Each wave takes its own 96 columns; the
//     two waves of a row group add their sums through LDS in a fixed order,
//     and the tile's sum is stored (no atomics) as this column tile's
//     partial, next_lora_part[tile, m, r]; a second kernel adds the tiles in
//     order;
//  3. lane l takes tile row l: the same x, nvfp4 per 16 columns
//     (nvfp4_quant16, the quantize kernel's reading); the next layer's
//     product operand e2m1 * dec(s8) as fp16 overwrites the lane's own tile
//     row, and the wave then stores the tile with consecutive lanes on
//     consecutive 16-byte pieces of a row.
// Columns past N have 1/smooth 0 (x = 0) and are not stored; rows past M are
// not stored.
// `xch` is LDS of 2 kWM 16 kXchRow floats, free during this epilogue.
__device__ __forceinline__ void gelu_quant_epilogue(const GemmArgs& args, f32x16 (&acc)[kIB][kJB], int m0, int n0,
                                                    int wave, int wm, int wn, int lane, int l32, int h,
                                                    const float* nmu, uint8_t* tile_base, float* xch,
                                                    bool add_bias) {
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
    const float bv = (add_bias && bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        *(uint16_t*)(gt + r * kGeluRow + (j * 32 + l32) * 2) = kGeluBf16[f32_to_bf16_bits(acc[i][j][e] + bv)];
      }
  }
  // (the wave's own LDS writes and reads execute in order)

  // 2 and 3 read the next layer's 1 / smooth of this wave's columns
  const float* mu = nmu + wn * (kJB * 32);
  // 2. the next layer's low-rank down projection of this wave's 96 columns
  // (its own GELU tile, in program order after step 1), 16 tile rows and 32
  // ranks at a time; the wave wn = 1 hands its sums to the wave wn = 0 of
  // its row group through `xch`, which adds them to its own (in that order)
  // and stores the column tile's partial.  xch alternates between two halves,
  // so one workgroup barrier per exchange suffices.
  const int nrank = args.next_rank;
  if (nrank > 0) {
    const int r16 = lane & 15, q = lane >> 4;
    const int nt = n0 / kBN;
    // next_lora_down [nrank, N]: reads past the end of the array return zero
    const __amdgpu_buffer_rsrc_t ld_rs = make_rsrc(args.next_lora_down, (size_t)nrank * N * 2);
    int parity = 0;
#pragma unroll 1
    for (int rc = 0; rc < nrank; rc += 32) {
#pragma unroll 1
      for (int rb = 0; rb < 4; ++rb, parity ^= 1) {
        bf16x8 ahi[kJB], alo[kJB];
#pragma unroll
        for (int ks = 0; ks < kJB; ++ks) {
          const u32x4 g = *(const u32x4*)(gt + (rb * 16 + r16) * kGeluRow + (ks * 32 + 8 * q) * 2);
          const f32x4 mu0 = *(const f32x4*)(mu + ks * 32 + 8 * q);
          const f32x4 mu1 = *(const f32x4*)(mu + ks * 32 + 8 * q + 4);
          u32x4 hi4, lo4;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float a = __fmul_rn(bf16_lo(g[p]), p < 2 ? mu0[2 * p] : mu1[2 * p - 4]);
            const float b = __fmul_rn(bf16_hi(g[p]), p < 2 ? mu0[2 * p + 1] : mu1[2 * p - 3]);
            const uint32_t hh = bf16x2_rne(a, b);
            hi4[p] = hh;
            lo4[p] = bf16x2_rne(__fsub_rn(a, bf16_lo(hh)), __fsub_rn(b, bf16_hi(hh)));
          }
          ahi[ks] = __builtin_bit_cast(bf16x8, hi4);
          alo[ks] = __builtin_bit_cast(bf16x8, lo4);
        }
        f32x4 d[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int rk = rc + 16 * h2;
          d[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (rk < nrank) {
#pragma unroll
            for (int ks = 0; ks < kJB; ++ks) {
              const bf16x8 b = __builtin_bit_cast(
                  bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                              ld_rs, ((rk + r16) * N + n0 + wn * (kJB * 32) + ks * 32 + 8 * q) * 2, 0, 0));
              d[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[ks], b, d[h2], 0, 0, 0);
              d[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], b, d[h2], 0, 0, 0);
            }
          }
        }
        // D: lane (c, q) holds rows 4q + j of the row block, rank column c
        float* xb = xch + (parity * kWM + wm) * (16 * kXchRow);
        if (wn == 1) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int j = 0; j < 4; ++j) xb[(4 * q + j) * kXchRow + 16 * h2 + r16] = d[h2][j];
        }
        lds_barrier();
        if (wn == 0) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int rk = rc + 16 * h2;
            if (rk >= nrank) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int m = m0 + wm * 64 + rb * 16 + 4 * q + j;
              const float v = __fadd_rn(d[h2][j], xb[(4 * q + j) * kXchRow + 16 * h2 + r16]);
              if (m < M) args.next_lora_part[((size_t)nt * M + m) * nrank + rk + r16] = v;
            }
          }
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
// the q | k heads 128 nt / D .. of this tile (head index below `heads`: q,
// else k), 128..191 v columns (qk_col).  Wave column group wn = 0 holds tile
// columns 0..95, wn = 1 columns 96..127 and the 64 v columns; a head may
// span both (D = 64: head 1 of the tile; D = 128: the only one).  Steps:
//  1. h = bf16(acc + bias) into the wave's LDS tile (rows of kGeluRow bytes);
//  2. lane l takes tile row l: the sums of squares of its columns of each
//     head; the two waves of a row block add theirs through LDS (`ssq`, in a
//     fixed order: wn = 0 first) and r = 1 / sqrt(sum / D + eps) per head;
//  3. each head pair (2i, 2i+1): n = bf16(fl32(fl32(h r) w_d)), then
//     (n_a cos - n_b sin, n_a sin + n_b cos) in fp32, rounded to bf16 in
//     place; v columns keep h;
//  4. the wave stores the tile with consecutive lanes on consecutive 16-byte
//     pieces of a row.
// Pieces of 8 columns never cross a head edge (D is a multiple of 8).  NH =
// 128 / D heads per tile, a compile-time constant.
template <int NH>
__device__ __forceinline__ void qk_norm_rope_epilogue(const GemmArgs& args, f32x16 (&acc)[kIB][kJB], int m0, int nt,
                                                      int wave, int wm, int wn, int lane, int l32, int h,
                                                      uint8_t* tile_base, float* ssq, bool add_bias) {
  const int M = (int)args.M, N = (int)args.N;
  const int heads = args.heads;
  constexpr int D = kQkCols / NH;
  const int qk_cols = 2 * heads * D;
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
    const float bv = (add_bias && bias) ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        *(uint16_t*)(gt + r * kGeluRow + (j * 32 + l32) * 2) = (uint16_t)f32_to_bf16_bits(acc[i][j][e] + bv);
      }
  }
  // (the wave's own LDS writes and reads execute in order)

  // 2. RMSNorm factors of the lane's row, one per head of the tile
  constexpr int kMaxHeads = NH;
  uint8_t* rowp = gt + lane * kGeluRow;
  const int c0 = wn * (kJB * 32);                            // tile column of the wave's first column
  const int nqk = wn == 0 ? kJB * 32 : kQkCols - kJB * 32;  // q | k columns of this wave (96 | 32)
  float ss[kMaxHeads];
#pragma unroll
  for (int hh = 0; hh < kMaxHeads; ++hh) ss[hh] = 0.f;
#pragma unroll
  for (int t = 0; t < 12; ++t) {
    if (8 * t < nqk) {
      const u32x4 v = *(const u32x4*)(rowp + 16 * t);
      const int hl = (c0 + 8 * t) / D;  // head of the tile
      float acc2 = 0.f;
#pragma unroll
      for (int hh = 0; hh < kMaxHeads; ++hh) acc2 = hh == hl ? ss[hh] : acc2;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = bf16_lo(v[p]), b = bf16_hi(v[p]);
        acc2 = __fmaf_rn(a, a, acc2);
        acc2 = __fmaf_rn(b, b, acc2);
      }
#pragma unroll
      for (int hh = 0; hh < kMaxHeads; ++hh) ss[hh] = hh == hl ? acc2 : ss[hh];
    }
  }
  const int trow = wm * 64 + lane;  // row of the workgroup tile
  constexpr int nh = NH;
#pragma unroll
  for (int hh = 0; hh < kMaxHeads; ++hh)
    if (hh < nh) ssq[(wn * kMaxHeads + hh) * kBM + trow] = ss[hh];
  lds_barrier();
  float rr[kMaxHeads];
  constexpr float invd = 1.0f / (float)D;  // exact: D is a power of two
#pragma unroll
  for (int hh = 0; hh < kMaxHeads; ++hh) {
    rr[hh] = 0.f;
    if (hh < nh) {
      const float tot = __fadd_rn(ssq[hh * kBM + trow], ssq[(kMaxHeads + hh) * kBM + trow]);
      rr[hh] = __fdiv_rn(1.0f, __fsqrt_rn(__fmaf_rn(tot, invd, args.eps)));
    }
  }

  // 3. normalize and rotate the head columns in place
  const int m = m0 + trow;
  const size_t trow_off = (size_t)min(m, M - 1) * (D / 2);
  const float* cs = args.rope_cos + trow_off;
  const float* sn = args.rope_sin + trow_off;
#pragma unroll
  for (int t = 0; t < 12; ++t) {
    if (8 * t < nqk) {
      const u32x4 v = *(const u32x4*)(rowp + 16 * t);
      const int tc = c0 + 8 * t;
      const int hl = tc / D;
      const int d = tc - hl * D;  // head dim of the piece's first column
      float r = 0.f;
#pragma unroll
      for (int hh = 0; hh < kMaxHeads; ++hh) r = hh == hl ? rr[hh] : r;
      // q heads come first in q | k
      const uint32_t* nw = (const uint32_t*)(nt * nh + hl < heads ? args.q_norm : args.k_norm);  // bf16 pairs
      const int pr = d >> 1;  // first pair of the piece
      const f32x4 c4 = *(const f32x4*)(cs + pr);
      const f32x4 s4 = *(const f32x4*)(sn + pr);
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t wp = nw[pr + p];
        const float na = __uint_as_float(f32_to_bf16_bits(__fmul_rn(__fmul_rn(bf16_lo(v[p]), r), bf16_lo(wp))) << 16);
        const float nb = __uint_as_float(f32_to_bf16_bits(__fmul_rn(__fmul_rn(bf16_hi(v[p]), r), bf16_hi(wp))) << 16);
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
  __shared__ float nmu[kBN];    // MLP fusion: 1 / smooth of the next layer for this tile's columns
  // int4 (fp8 operands): the group scales of the stages in LDS, A per pair
  // of stages [stage of the pair][row] (the bf16 scales of the row's two
  // groups in one word), W [stage % 3][group][row]
  constexpr bool kFp8 = PREC == kInt4 && !PARTIALS;
  // (one object per pair of stages in flight, as for the A buffers: a read of
  // one does not wait for the direct-to-LDS loads still filling another)
  __shared__ __attribute__((aligned(16))) uint32_t asc0[kFp8 ? 2 * kBM : 1];
  __shared__ __attribute__((aligned(16))) uint32_t asc1[kFp8 ? 2 * kBM : 1];
  __shared__ __attribute__((aligned(16))) uint32_t asc2[kFp8 ? 2 * kBM : 1];
  // (W: bf16 bits of s_w / 2, the operand of the scale-product instruction,
  // [stage % 3][group][row])
  __shared__ __attribute__((aligned(16))) uint16_t wsc[kFp8 ? 3 * 2 * kBN : 1];
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
  // (a stage is kBK values of K; the int4 fp8 path takes two groups, 128)
  int s0 = 0, nstages = kFp8 ? K / 128 : K / kBK;
  if constexpr (kSplit) {
    const int per = (nstages + args.ksplit - 1) / args.ksplit;
    s0 = blockIdx.y * per;
    nstages = min(per, nstages - s0);
  }
  // physical column of tile column c (the QKV fusion reorders columns)
  constexpr bool kQk = EPI == kEpiQk;
  const int qk_cols = kQk ? 2 * args.heads * args.head_dim : 0;
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
  f32x16 acc[kIB][kJB];
#pragma unroll
  for (int i = 0; i < kIB; ++i)
#pragma unroll
    for (int j = 0; j < kJB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- low-rank up: acc += (lora_act_hi + lora_act_lo) lora_up^T -------------
  // (split K: in split 0 only).  The int4 path runs it first, while the
  // loads of its first stages are in flight; nvfp4 runs it after the main
  // loop, whose sum is first multiplied by the weight tensor scale.
  const bool lora_here = !kSplit || blockIdx.y == 0;
  auto lora_load = [&](int rs16, LoraOps& o) {
    constexpr int rank = RB * 16;
    const uint16_t* __restrict__ lu = (const uint16_t*)args.lora_up;
#pragma unroll
    for (int i = 0; i < kIB; ++i) {
      const int row = min(m0 + wm * (kIB * 32) + i * 32 + l32, M - 1);
      const float* la = args.lora_act + (size_t)row * rank + rs16 * 16 + h * 8;
      o.a[i][0] = *(const f32x4*)la;
      o.a[i][1] = *(const f32x4*)(la + 4);
    }
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      const int tc = wn * (kJB * 32) + j * 32 + l32;
      const int col = kQk ? pcol(tc) : min(n0 + tc, N - 1);
      o.b[j] = *(const u32x4*)(lu + (size_t)col * rank + rs16 * 16 + h * 8);
    }
  };
  auto lora_mma = [&](const LoraOps& o) {
    bf16x8 ahi[kIB], alo[kIB];
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = o.a[i][e >> 2][e & 3];
        const __bf16 hb = (__bf16)v;
        ahi[i][e] = hb;
        alo[i][e] = (__bf16)(v - (float)hb);
      }
#pragma unroll
    for (int i = 0; i < kIB; ++i)
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        const bf16x8 bo = __builtin_bit_cast(bf16x8, o.b[j]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[i], bo, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[i], bo, acc[i][j], 0, 0, 0);
      }
  };
  auto lowrank_up = [&]() {
    if constexpr (RB > 0 && !PARTIALS) {
      if (lora_here) {
#pragma unroll
        for (int rs16 = 0; rs16 < RB; ++rs16) {
          LoraOps o;
          lora_load(rs16, o);
          lora_mma(o);
        }
      }
    }
  };

  if constexpr (kFp8) {
    // ---- int4: fp8 operands, group scales per group ----------------------------
    // A stage s (128 values of K, two groups of 64) comes straight from
    // memory to LDS as fp8 codes in the same swizzled 16-byte chunks as the
    // fp16 operand of the other path (8 chunks per 128-byte row); its group
    // scales (bf16 [M, K/64]) likewise, two stages per load, into asc0-2.
    // W stage s is staged
    // through registers: int4 nibbles -> fp8 bytes (rows of kWRow bytes),
    // its bf16 group scales halved -> wsc.  Per group, each 32 x 32 tile is
    // one v_mfma_f32_32x32x64_f8f6f4 of exact integer sums P (|P| <= 64 * 49),
    // one bf16 outer product of the scales, and acc += P * (s_x * s_w) (the
    // scale product is exact in fp32).
    // Loads run three stages ahead for A and two for W, as in the other path.
    const int G = K >> 6;
    const __amdgpu_buffer_rsrc_t a_rs = make_rsrc((const uint8_t*)args.act + (size_t)m0 * K + s0 * 128,
                                                  (size_t)(M - m0) * K - s0 * 128);
    const __amdgpu_buffer_rsrc_t as_rs = make_rsrc((const uint8_t*)args.act_scale + ((size_t)m0 * G + 2 * s0) * 2,
                                                   ((size_t)(M - m0) * G - 2 * s0) * 2);
    const int w_base = kQk ? 0 : n0;
    const __amdgpu_buffer_rsrc_t w_rs = make_rsrc((const uint8_t*)args.w_codes + (size_t)w_base * K2 + s0 * 64,
                                                  (size_t)(N - w_base) * K2 - s0 * 64);
    const __amdgpu_buffer_rsrc_t ws_rs = make_rsrc((const uint8_t*)args.w_scales + (size_t)w_base * G * 2 + s0 * 4,
                                                   (size_t)(N - w_base) * G * 2 - s0 * 4);
    const __amdgpu_buffer_rsrc_t zero_rs = make_rsrc(args.w_codes, 0);
    // W codes: rows 0-127 of the tile 16 bytes per thread, rows 128-191 8
    // bytes (fewer load instructions per stage than three 8-byte pieces)
    const int la_r = tid >> 2, la_c = tid & 3, lb_r = 2 * kRP + (tid >> 3), lb_c = tid & 7;
    const int wa_off = (kQk ? pcol(la_r) : la_r) * K2 + la_c * 16;  // rows from the descriptor base
    const int wb_off = (kQk ? pcol(lb_r) : lb_r) * K2 + lb_c * 8;
    // W scales: wave w loads those of tile rows 24 w .. 24 w + 23, one row
    // per lane, one load per wave and pair of stages (even s): lanes 0-23
    // stage s, lanes 24-47 stage s + 1, lanes 48-63 repeat lanes 0-15.  (At
    // an odd stage count the last pair's second half lies past the last
    // stage: the next split's or the next row's scales, never used, or
    // beyond the descriptor, zero.)
    const int srow = wave * (kBN / kWaves) + lane % (kBN / kWaves);
    const int s_next = (lane >= kBN / kWaves && lane < 2 * (kBN / kWaves)) ? 1 : 0;
    const int ws_off = (kQk ? pcol(srow) : srow) * G * 2 + s_next * 4;
    int dma_off[kADma];
#pragma unroll
    for (int d = 0; d < kADma; ++d) {
      const int u = (wave * kADma + d) * 64 + lane;
      const int row = u >> 3;
      dma_off[d] = row * K + a_pos(row, u & 7) * 16;
    }
    // A scales, one load per pair of stages (s even): waves 0-3 load the
    // two groups of stage s, waves 4-7 those of stage s + 1, one row per lane
    // (4 bytes).  (At an odd stage count the last pair's second stage is the
    // next split's first or the next row's first, never used, or beyond the
    // descriptor, zero.)
    const int sc_row = (wave & 3) * 64 + lane, sc_st = wave >> 2;
    const int sc_off = sc_row * G * 2 + sc_st * 4;

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
    // the A scale object of stage s (st = s % 6): pair st / 2
    auto ascbuf = [&](auto st) -> uint32_t* {
      constexpr int i = decltype(st)::value % 6 / 2;
      if constexpr (i == 0) return asc0;
      else if constexpr (i == 1) return asc1;
      else return asc2;
    };
    // loads of stage s (st = s % 6): A into A buffer s % 3 (direct to LDS),
    // with the A scales of stages s and s + 1 if s is even, then W into r
    // (with the W scales of stages s and s + 1 if s is even)
    auto group = [&](RawStage8& r, int s, auto st) {
      constexpr int q = decltype(st)::value;
      const bool live = s < nstages;
      uint8_t* dst = abuf(st) + wave * (kADma * 64 * 16);
#pragma unroll
      for (int d = 0; d < kADma; ++d)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? a_rs : zero_rs,
                                                 (__attribute__((address_space(3))) void*)(dst + d * 1024), 16,
                                                 dma_off[d], s * 128, 0, 0);
      if constexpr (q % 2 == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            live ? as_rs : zero_rs,
            (__attribute__((address_space(3))) void*)(ascbuf(st) + sc_st * kBM + (wave & 3) * 64), 4, sc_off,
            s * 4, 0, 0);
      // the W loads of the stage stay behind its A loads: a wave that has
      // waited for its W registers has also received its A stage
      __builtin_amdgcn_sched_barrier(0);
      r.wa = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(live ? w_rs : zero_rs, wa_off, s * 64, 0));
      r.wb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(live ? w_rs : zero_rs, wb_off, s * 64, 0));
      if constexpr (q % 2 == 0)
        r.sw = __builtin_amdgcn_raw_buffer_load_b32(live ? ws_rs : zero_rs, ws_off, s * 4, 0);
    };
    // staging of third p of raw stage st (mod 6) into W buffer Tw (the two
    // halves of wa, then wb; with part 0 of an even stage, the wave's W
    // scales of stages st and st + 1 into wsc slots st % 3 and (st + 1) % 3)
    auto store_part = [&](uint8_t* Tw, auto st, const RawStage8& r, int p) {
      constexpr int q = decltype(st)::value;
      if (p < 2)
        *(u32x4*)(Tw + la_r * kWRow + la_c * 32 + p * 16) = int4x16_to_fp8(u32x2{r.wa[2 * p], r.wa[2 * p + 1]});
      else
        *(u32x4*)(Tw + lb_r * kWRow + lb_c * 16) = int4x16_to_fp8(r.wb);
      if (q % 2 == 0 && p == 0) {
        // s_w / 2 as bf16 (exact: a power-of-two step of a normal value);
        // lanes holding the same row and stage write the same values
        uint16_t* d = wsc + (q % 3) * 2 * kBN + srow + (q % 3 == 2 ? -2 : 1) * (s_next * 2 * kBN);
        d[0] = (uint16_t)(__float_as_uint(__fmul_rn(bf16_lo(r.sw), 0.5f)) >> 16);
        d[kBN] = (uint16_t)(__float_as_uint(__fmul_rn(bf16_hi(r.sw), 0.5f)) >> 16);
      }
    };
    // one stage: per group, per 32 x 32 tile one product of 64 values of K
    auto compute = [&](auto P, int s, RawStage8& r) {
      constexpr int p = decltype(P)::value;
      constexpr int ab = p % kAStages;
      const uint8_t* Ta = abuf(IC<p>{});
      const uint8_t* Tw = wbuf(IC<p>{});
      uint8_t* Nw = wbuf(IC<p + 1>{});
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        i32x8 aop[kIB], bop[kJB];
        // the scale products s_x s_w of a 32 x 32 block come from one bf16
        // instruction of K = 8 (an outer product): element 0 of each lane's
        // four values of K is s_x (A, row l32 of block i) or s_w / 2 (B,
        // column l32 of block j), the rest zero; lanes 32-63 (K = 4..7)
        // repeat them, so D = 2 (s_x s_w / 2) = s_x s_w, exact in fp32
        uint32_t as16[kIB], bs16[kJB];
#pragma unroll
        for (int i = 0; i < kIB; ++i) {
          const int row = wm * (kIB * 32) + i * 32 + l32;
          const u32x4 lo = *(const u32x4*)(Ta + row * kARow + a_pos(row, 4 * gi + 2 * h) * 16);
          const u32x4 hi = *(const u32x4*)(Ta + row * kARow + a_pos(row, 4 * gi + 2 * h + 1) * 16);
          aop[i] = __builtin_bit_cast(i32x8, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          // the bf16 scale of group gi of the row
          as16[i] = ((const uint16_t*)(ascbuf(IC<p>{}) + (p % 2) * kBM + row))[gi];
        }
#pragma unroll
        for (int j = 0; j < kJB; ++j) {
          const int col = wn * (kJB * 32) + j * 32 + l32;
          const uint8_t* src = Tw + col * kWRow + 64 * gi + 32 * h;
          const u32x4 lo = *(const u32x4*)src, hi = *(const u32x4*)(src + 16);
          bop[j] = __builtin_bit_cast(i32x8, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          bs16[j] = wsc[((p % 3) * 2 + gi) * kBN + col];
        }
#pragma unroll
        for (int i = 0; i < kIB; ++i) {
#pragma unroll
          for (int j = 0; j < kJB; ++j) {
            const f32x16 pr = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[i], bop[j], f32x16{}, 0, 0, 0, 0,
                                                                            0, 0);
            const f32x16 sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(
                __builtin_bit_cast(s16x4, u32x2{as16[i], 0u}), __builtin_bit_cast(s16x4, u32x2{bs16[j], 0u}), f32x16{},
                0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = __fmaf_rn(pr[e], sc[e], acc[i][j][e]);
          }
          // stage a third of the next W stage among the products
          if (gi * kIB + i < 3) store_part(Nw, IC<(p + 1) % 6>{}, r, gi * kIB + i);
          // order of a tile row's instructions: the products of two blocks,
          // the scaling of the first, the third block's products, the rest
          // (62.5 us against 63.5 us in the compiler's own order at M = 4096,
          // K = N = 3072)
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
        }
      }
      stage_barrier();
      group(r, s + 3, IC<(p + 3) % 6>{});
    };

    // Prologue.  The bias (except for split-K partials) and, for ranks up to
    // 32, the low-rank operands are requested before the first stages, so
    // that the wait for them is not a wait for the stages; the sum starts
    // from the bias, then adds the low rank, then the groups (the epilogues
    // add no bias on this path).
    constexpr bool kLoraFirst = RB > 0 && RB <= 2;
    LoraOps lops[kLoraFirst ? RB : 1];
    if constexpr (kLoraFirst) {
      if (lora_here) {
#pragma unroll
        for (int rs16 = 0; rs16 < RB; ++rs16) lora_load(rs16, lops[rs16]);
      }
    }
    float bv[kJB];
    if constexpr (!kSplit) {
      const uint16_t* bias = (const uint16_t*)args.bias;
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        const int col = pcol(wn * (kJB * 32) + j * 32 + l32);
        bv[j] = (bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.f;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    RawStage8 r0, r1;
    group(r0, 0, IC<0>{});
    group(r1, 1, IC<1>{});
    if constexpr (!kSplit) {
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int j = 0; j < kJB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = bv[j];
    }
    if constexpr (kLoraFirst) {
      if (lora_here) {
#pragma unroll
        for (int rs16 = 0; rs16 < RB; ++rs16) lora_mma(lops[rs16]);
      }
    } else {
      lowrank_up();
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) store_part(lds_w0, IC<0>{}, r0, q);
    group(r0, 2, IC<2>{});
    stage_barrier();  // (each wave has its stage-0 A loads: they precede the W loads it staged)
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
  } else {
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
  // nvfp4 linear: tile rows 0-127 by one 8-byte load (one scale block) per
  // thread and stage, rows 128-191 as piece 2 (fewer load instructions)
  constexpr bool kW8 = PREC == kNvfp4 && !PARTIALS;
  const int la_r = tid >> 2, la_c = tid & 3;
  const int wa_row = kQk ? pcol(la_r) : la_r;
  const int wa_off = wa_row * K2 + la_c * 8, wsa_off = wa_row * (int)ws_row_bytes;
  const int wsb_off = (kQk ? pcol(lr + 2 * kRP) : lr + 2 * kRP) * (int)ws_row_bytes;
  const int sp_b4 = s0 > 0 ? 4 : 0;
  const __amdgpu_buffer_rsrc_t wsp_rs =
      make_rsrc((const uint8_t*)args.w_scales + (size_t)w_base * ws_row_bytes + ws_s0 - sp_b4,
                kW8 ? (size_t)(N - w_base) * ws_row_bytes - ws_s0 + sp_b4 : 0);
  // (the scale bytes of the odd stage of a pair, taken out at the even one)
  uint32_t nsc_a = 0, nsc_b = 0;
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

  // loads of stage s: A into A buffer ab (direct to LDS), W into r (par:
  // s % 2)
  auto group = [&](RawStage& r, int s, auto ab, auto par) {
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
    if constexpr (kW8) {
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wrs, wa_off, s * 32, 0));
      r.w[0] = v[0];
      r.w[1] = v[1];
      if constexpr (decltype(par)::value == 0) {
        // the scales of stages s and s + 1 (8 bytes of the row); when s is
        // the last stage (an odd stage count, split K only: K / 64 is even),
        // those of s - 1 and s, so that the load stays inside the row (the
        // pair descriptor starts one stage before s0 when s0 > 0)
        const int so = (s + 1 == nstages && (s > 0 || s0 > 0) ? s - 1 : s) * 4 + sp_b4;
        const __amdgpu_buffer_rsrc_t prs = live ? wsp_rs : zero_rs;
        r.spa = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(prs, wsa_off, so, 0));
        r.w[2] = __builtin_amdgcn_raw_buffer_load_b32(wrs, w_off[2], s * 32, 0);
        r.spb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(prs, wsb_off, so, 0));
      } else {
        r.w[2] = __builtin_amdgcn_raw_buffer_load_b32(wrs, w_off[2], s * 32, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kWP; ++j) {
        r.w[j] = __builtin_amdgcn_raw_buffer_load_b32(wrs, w_off[j], s * 32, 0);
        if constexpr (PREC == kNvfp4 && !PARTIALS) r.sw8[j] = __builtin_amdgcn_raw_buffer_load_b8(srs, ws_off[j], s * 4, 0);
      }
    }
    if constexpr (PARTIALS) {
#pragma unroll
      for (int i = 0; i < kAP; ++i) r.a[i] = __builtin_amdgcn_raw_buffer_load_b32(ars, pa_off[i], s * 32, 0);
    }
  };

  // staging of one raw stage q (par: q % 2) in three parts (part p: W piece p
  // and, for the parity export, A pieces of part p), so that it can be
  // interleaved with the matrix instructions of the previous stage
  auto store_part = [&](uint8_t* Ta, uint8_t* Tw, const RawStage& r, int p, auto par, int q) {
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
    if constexpr (kW8) {
      // pieces 0 and 1: columns 16c .. 16c+7 and 16c+8 .. 16c+15 of row tid/4
      // (scale byte c of the row's stage), piece 2 as the other paths
      // (scale byte c / 2)
      const int sh = 8 * (p < 2 ? la_c : (lc >> 1));
      uint32_t sb;
      if constexpr (decltype(par)::value == 0) {
        const u32x2 sp = p < 2 ? r.spa : r.spb;
        sb = ((q + 1 == nstages && (q > 0 || s0 > 0) ? sp[1] : sp[0]) >> sh) & 0xFFu;
        if (p == 0) nsc_a = (sp[1] >> sh) & 0xFFu;
        if (p == 2) nsc_b = (sp[1] >> sh) & 0xFFu;
      } else {
        sb = p < 2 ? nsc_a : nsc_b;
      }
      const _Float16 sc = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sb, 0);
      uint8_t* dst = p < 2 ? Tw + la_r * kWRow + la_c * 32 + p * 16 : Tw + (lr + 2 * kRP) * kWRow + lc * 16;
      *(f16x8*)dst = e2m1x8_to_f16_scaled(r.w[p], sc);
    } else {
      const int wrow = lr + kRP * p;
      _Float16 sc = (_Float16)(PREC == kInt4 ? 1.0f : 2.0f);
      if constexpr (!PARTIALS) sc = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)r.sw8[p], 0);  // nvfp4
      *(f16x8*)(Tw + wrow * kWRow + lc * 16) =
          PREC == kInt4 ? int4x8_to_f16_scaled(r.w[p], sc) : e2m1x8_to_f16_scaled(r.w[p], sc);
    }
  };

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
      if (ks < 3) store_part(Na, Nw, r, ks, IC<(p + 1) % 2>{}, s + 1);
      if (ks == 3) group(r, s + 3, IC<p>{}, IC<(p + 1) % 2>{});
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
  group(r0, 0, IC<0>{}, IC<0>{});
  group(r1, 1, IC<1>{}, IC<1>{});
#pragma unroll
  for (int p = 0; p < 3; ++p) store_part(lds_a0, lds_w0, r0, p, IC<0>{}, 0);
  group(r0, 2, IC<2>{}, IC<0>{});
  stage_barrier();  // (each wave has its stage-0 A loads: they precede the W loads it staged)
  rd(lds_a0, lds_w0, 0, 0);
  // Six stages per iteration (the A ring of three times the two raw register
  // stages), all straight-line code.  Stages past the last (up to five when
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
  }

  if constexpr (!PARTIALS) {
    // ---- nvfp4: the weight tensor scale (int4 applied its scales per group) --
    if constexpr (PREC == kNvfp4) {
      const float t = args.wtscale;
#pragma unroll
      for (int i = 0; i < kIB; ++i)
#pragma unroll
        for (int j = 0; j < kJB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = __fmul_rn(acc[i][j][e], t);
    }
    // ---- low-rank up (int4: done before the main loop) -----------------------
    if constexpr (!kFp8) lowrank_up();
    if constexpr (EPI == kEpiGelu) {
      // tile of wave w: base (w < 2: a0, < 4: a1, < 6: a2, else w0) + (w & 1) 64 rows
      gelu_quant_epilogue(args, acc, m0, n0, wave, wm, wn, lane, l32, h, nmu,
                          wave < 2 ? lds_a0 : wave < 4 ? lds_a1 : wave < 6 ? lds_a2 : lds_w0, (float*)lds_w1, !kFp8);
    } else if constexpr (kQk) {
      uint8_t* tb = wave < 2 ? lds_a0 : wave < 4 ? lds_a1 : wave < 6 ? lds_a2 : lds_w0;
      if (args.head_dim == 128)
        qk_norm_rope_epilogue<1>(args, acc, m0, nt, wave, wm, wn, lane, l32, h, tb, (float*)lds_w1, !kFp8);
      else if (args.head_dim == 64)
        qk_norm_rope_epilogue<2>(args, acc, m0, nt, wave, wm, wn, lane, l32, h, tb, (float*)lds_w1, !kFp8);
      else
        qk_norm_rope_epilogue<4>(args, acc, m0, nt, wave, wm, wn, lane, l32, h, tb, (float*)lds_w1, !kFp8);
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
      // ---- bias + bf16 store, through a wave-private LDS tile -----------------
      // (the wave's 64 x 96 block is written to LDS in the matrix layout and
      // stored with consecutive lanes on consecutive 16-byte pieces of a row)
      uint8_t* gt = (wave < 2 ? lds_a0 : wave < 4 ? lds_a1 : wave < 6 ? lds_a2 : lds_w0) + (wave & 1) * (64 * kGeluRow);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, expcnt 7, lgkmcnt 0
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const uint16_t* bias = (const uint16_t*)args.bias;
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        const int col = n0 + wn * (kJB * 32) + j * 32 + l32;
        // (int4: the sum started from the bias)
        const float bv = (!kFp8 && bias && col < N) ? bf16_bits_to_f32(bias[col]) : 0.f;
#pragma unroll
        for (int i = 0; i < kIB; ++i)
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            // rows r and r + 1 of the lane's column, one packed RNE conversion
            const int r = i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
            const float v0 = kFp8 ? acc[i][j][e] : acc[i][j][e] + bv;
            const float v1 = kFp8 ? acc[i][j][e + 1] : acc[i][j][e + 1] + bv;
            const uint32_t pk = bf16x2_rne(v0, v1);
            *(uint16_t*)(gt + r * kGeluRow + (j * 32 + l32) * 2) = (uint16_t)pk;
            *(uint16_t*)(gt + (r + 1) * kGeluRow + (j * 32 + l32) * 2) = (uint16_t)(pk >> 16);
          }
      }
      const int c0 = n0 + wn * (kJB * 32);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        const int c = 64 * i + lane;
        const int r = c / 12, k = c - 12 * r;
        const u32x4 v = *(const u32x4*)(gt + r * kGeluRow + 16 * k);
        const int m = m0 + wm * 64 + r;
        if (m < M && c0 + 8 * k < N) *(u32x4*)((uint16_t*)args.out + (size_t)m * N + c0 + 8 * k) = v;
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
// added in order (deterministic); 8 columns per thread (N % 64 == 0).  The
// loads of all splits (at most kMaxSplit) are issued before the additions.
constexpr int kMaxSplit = 8;
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int ksplit, int64_t M,
                                                            int64_t N, const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;  // first element
  if (i >= M * N) return;
  const int64_t n = i % N;
  f32x4 a[kMaxSplit], b[kMaxSplit];
#pragma unroll
  for (int j = 0; j < kMaxSplit; ++j) {
    if (j < ksplit) {
      const f32x4* p = (const f32x4*)(partial + (size_t)j * M * N + i);
      a[j] = __builtin_nontemporal_load(p);
      b[j] = __builtin_nontemporal_load(p + 1);
    }
  }
  const u32x4 bb = bias ? *(const u32x4*)(bias + n) : u32x4{0u, 0u, 0u, 0u};
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxSplit; ++j) {
    if (j < ksplit) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] += a[j][c];
        acc[4 + c] += b[j][c];
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float b0 = bf16_bits_to_f32((uint16_t)(bb[c] & 0xFFFFu));
    const float b1 = bf16_bits_to_f32((uint16_t)(bb[c] >> 16));
    o[c] = f32_to_bf16_bits(acc[2 * c] + b0) | (f32_to_bf16_bits(acc[2 * c + 1] + b1) << 16);
  }
  *(u32x4*)(out + i) = o;
}

// out[i] = sum_t part[t, i], t = 0 .. tiles-1 in order (the fused MLP's
// low-rank activations of the down layer from the up projection's column
// tiles).  A thread sums four consecutive floats; the loads of eight tiles
// are issued before their additions, which stay in tile order.
__global__ __launch_bounds__(64) void tile_partial_sum_kernel(const float* __restrict__ part, int tiles, int64_t n4,
                                                              float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = (const f32x4*)part + i;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  int t = 0;
  for (; t + 8 <= tiles; t += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + (size_t)(t + u) * n4);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = __fadd_rn(a[c], v[u][c]);
  }
  for (; t < tiles; ++t) {
    const f32x4 v = __builtin_nontemporal_load(p + (size_t)t * n4);
#pragma unroll
    for (int c = 0; c < 4; ++c) a[c] = __fadd_rn(a[c], v[c]);
  }
  ((f32x4*)out)[i] = a;
}

// n must be a multiple of 4 (M * rank, rank a multiple of 16)
hipError_t launch_tile_partial_sum(const float* part, int tiles, int64_t n, float* out, hipStream_t stream) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(tile_partial_sum_kernel, dim3((unsigned)((n4 + 63) / 64)), dim3(64), 0, stream, part, tiles, n4,
                     out);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N, const void* bias, void* out,
                                hipStream_t stream) {
  if (ksplit < 1 || ksplit > kMaxSplit) return hipErrorInvalidValue;
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
