// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

constexpr int kInt4 = 0;
constexpr int kNvfp4 = 1;

struct QuantActArgs {
  const void* x;          // bf16 [M, K]
  const void* smooth;     // bf16 [K]
  const void* lora_down;  // bf16 [rank, K]
  void* codes;            // parity export: u8 [M, K/2] nibbles; else null
  void* scales;           // parity export: bf16 [M, K/64] | u8 [M, K/16]; else null
  float* lora_act;        // f32 [M, rank]
  void* act_op;           // linear only: the product operand [M, K] (see below), else null
  float* act_scale;       // linear int4 only: [M, K/64] group scales s, f32 (the
                          // operand export) or bf16 bits (scale_bf16, the linear)
  int64_t M, K;
  int precision, rank;
  // linear only: K slices (1: one workgroup per 16 rows and all of K; S > 1:
  // S workgroups per 16 rows, each a K/S slice, the low-rank sums written as
  // fp32 partials lora_part [S, M, rank] for a second kernel to add in order)
  int k_slices = 1;
  float* lora_part = nullptr;
  // linear int4: write the group scales as their bf16 bits (they are bf16
  // values), the form the product kernel loads
  bool scale_bf16 = false;
};

// The product operand of the linear.  int4: the codes q (|q| <= 7) as fp8
// E4M3 bytes (every such integer is exact), with the group scales in
// act_scale (bf16 bits), applied after each group's product; nvfp4:
// e2m1 * dec(s8) as fp16 (always exact).

struct GemmArgs {
  const void* act;          // linear: act_op above; partials: nibbles [M, K/2]
  const uint16_t* act_scale;  // linear int4: bf16 [M, K/64]; else null
  const float* lora_act;    // f32 [M, rank]
  const void* w_codes;      // u8 [N, K/2]
  const void* w_scales;     // bf16 [N, K/64] | u8 [N, K/16]
  const void* lora_up;      // bf16 [N, rank]
  const void* bias;         // bf16 [N] or null
  void* out;                // bf16 [M, N]
  int32_t* partials;        // parity export: i32 [M, N, K/G] (then out is unused)
  float wtscale;
  int64_t M, K, N;
  int precision, rank;
  // MLP fusion (null next_act: plain store of out).  The epilogue applies
  // GELU to the bf16 output and quantizes it (nvfp4) for the next layer,
  // whose input channels are this layer's N columns; out is not written.
  const void* next_smooth = nullptr;     // bf16 [N]
  const void* next_lora_down = nullptr;  // bf16 [next_rank, N] or null
  void* next_act = nullptr;              // f16 [M, N]: the next layer's product operand e2m1 * dec(s8)
  float* next_lora_part = nullptr;       // f32 [column tiles, M, next_rank]: each tile's partial sum
  int next_rank = 0;
  // QKV fusion (heads > 0): N = 3 heads head_dim columns q | k | v, head_dim
  // 32, 64 or 128.  Column tile t of the heads head_dim / 64 tiles computes
  // the q | k columns 128 t .. 128 t + 127 (whole heads) and the v columns
  // 64 t .. 64 t + 63; the epilogue applies RMSNorm and RoPE to the heads.
  const void* q_norm = nullptr;     // bf16 [head_dim]
  const void* k_norm = nullptr;     // bf16 [head_dim]
  const float* rope_cos = nullptr;  // f32 [M, head_dim / 2]
  const float* rope_sin = nullptr;  // f32 [M, head_dim / 2]
  float eps = 0.f;
  int heads = 0;
  int head_dim = 0;
  // split K (ksplit > 1, plain linear only): workgroup (tile, j) covers stages
  // [j per, (j + 1) per) and writes fp32 partials [ksplit, M, N] (the low-rank
  // term in split 0, no bias); launch_splitk_reduce sums them into out
  int ksplit = 1;
  float* partial = nullptr;
};

struct AwqArgs {
  const void* x;        // bf16 [M, K]
  const void* w_codes;  // u8 [N, K/2]
  const void* scales;   // bf16 [N, K/64]
  const void* zeros;    // bf16 [N, K/64]
  const void* bias;     // bf16 [N] or null
  void* out;            // bf16 [M, N]
  int64_t M, K, N;
};

// Offline weight preparation (weight_prep.hip).
struct SmoothArgs {
  const void* x;   // bf16 [M, K] calibration activations
  const float* w;  // f32 [N, K] weight
  void* smooth;    // out: bf16 [K]
  uint32_t* amax;  // scratch: u32 [2 K]
  int64_t M, N, K;
};

struct PackArgs {
  const float* resid;  // f32 [N, K] residual weight
  void* packed;        // out: u8 [N, K/2]
  void* scales;        // out: bf16 [N, K/64] | u8 [N, K/16]
  float* wtscale;      // out: f32 [1] (1 for int4); may be null
  uint32_t* amax;      // scratch: u32 [1]
  int64_t N, K;
  int precision;
};

// Low-rank split of the weight preparation (prep_svd.hip).  A matrix operand
// of the products: the smoothed weight w[n, k] * smooth[k] (w non-null) or a
// dense row-major fp64 matrix.
struct PrepSrc {
  const float* w = nullptr;       // fp32 [R, C]
  const void* smooth = nullptr;   // bf16 [C]
  const double* dense = nullptr;  // fp64 [R, C] when w is null
};
constexpr int kPrepMaxL = 160;  // widest product (rank + oversampling)
hipError_t launch_prep_gauss(double* omega, int64_t n, uint64_t seed, hipStream_t s);
// out [R, l] = A [R, C] B [C, l]
hipError_t launch_prep_ab(const PrepSrc& a, int64_t R, int64_t C, const double* B, int l, double* out,
                          hipStream_t s);
// out [C, l] = A^T B, A [R, C], B [R, l]; part: fp64 [slices, C, l] scratch
hipError_t launch_prep_atb(const PrepSrc& a, int64_t R, int64_t C, const double* B, int l, int slices, double* part,
                           double* out, hipStream_t s);
hipError_t launch_prep_to_bf16(const double* src, int64_t rows, int64_t cols, int64_t ld, bool transpose,
                               uint16_t* dst, hipStream_t s);
hipError_t launch_prep_residual(const float* w, const void* smooth, const void* up, const void* down, int64_t N,
                                int64_t K, int rank, float* resid, hipStream_t s);

hipError_t launch_smooth_factors(const SmoothArgs& a, hipStream_t stream);
hipError_t launch_pack_weight(const PackArgs& a, hipStream_t stream);
hipError_t launch_quantize_act(const QuantActArgs& a, hipStream_t stream);
hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream);
// out[m, n] = bf16(sum_j partial[j, m, n] + bias[n]), j in order
hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N, const void* bias, void* out,
                                hipStream_t stream);
hipError_t launch_gelu_table_copy(uint16_t* out, hipStream_t stream);
// out[i] = sum_t part[t, i] over t = 0 .. tiles-1 in order, i < n
hipError_t launch_tile_partial_sum(const float* part, int tiles, int64_t n, float* out, hipStream_t stream);
hipError_t launch_awq_gemv(const AwqArgs& a, hipStream_t stream);

}  // namespace svdq
