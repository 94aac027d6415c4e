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
  void* act_f16;          // linear only: f16 [M, K] product operand q * s (see below), else null
  float* row_scale;       // linear int4 only: f32 [M] power-of-two factor of each row of act_f16
  int64_t M, K;
  int precision, rank;
  float* clear = nullptr;  // optional: f32 [clear_n] set to zero by the same launch (the fused
  int64_t clear_n = 0;     // MLP's accumulator for the next layer's low-rank activations)
};

// act_f16 holds the dequantized activations exactly: int4 q * s * 2^-E[m]
// (E[m] chosen per row so every value fits fp16, row_scale[m] = 2^E[m]);
// nvfp4 e2m1 * dec(s8), which always fits fp16.

struct GemmArgs {
  const void* act;          // linear: f16 [M, K] (act_f16 above); partials: nibbles [M, K/2]
  const float* row_scale;   // linear int4: f32 [M]; else null
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
  float* next_lora_act = nullptr;        // f32 [M, next_rank], zero on entry, accumulated with atomics
  int next_rank = 0;
  // QKV fusion (heads > 0): N = 3 heads 128 columns q | k | v.  Column tile t
  // of the 2 heads tiles computes head t of q | k and v columns 64 t ..
  // 64 t + 63; the epilogue applies RMSNorm and RoPE to the head's columns.
  const void* q_norm = nullptr;     // bf16 [128]
  const void* k_norm = nullptr;     // bf16 [128]
  const float* rope_cos = nullptr;  // f32 [M, 64]
  const float* rope_sin = nullptr;  // f32 [M, 64]
  float eps = 0.f;
  int heads = 0;
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

hipError_t launch_smooth_factors(const SmoothArgs& a, hipStream_t stream);
hipError_t launch_pack_weight(const PackArgs& a, hipStream_t stream);
hipError_t launch_quantize_act(const QuantActArgs& a, hipStream_t stream);
hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream);
// out[m, n] = bf16(sum_j partial[j, m, n] + bias[n]), j in order
hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N, const void* bias, void* out,
                                hipStream_t stream);
hipError_t launch_gelu_table_copy(uint16_t* out, hipStream_t stream);
hipError_t launch_awq_gemv(const AwqArgs& a, hipStream_t stream);

}  // namespace svdq
