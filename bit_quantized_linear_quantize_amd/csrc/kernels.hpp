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
  void* codes;            // u8 [M, K/2] nibbles, or (int4, fp8_codes) E4M3 [M, K]
  void* scales;           // bf16 [M, K/64] | u8 [M, K/16]
  float* lora_act;        // f32 [M, rank]
  int64_t M, K;
  int precision, rank;
  bool fp8_codes;         // int4 only: write E4M3 bytes in expansion order
};

struct GemmArgs {
  const void* act_codes;   // int4: E4M3 [M, K] (expansion order), or nibbles [M, K/2]
                           // when computing partials; nvfp4: nibbles [M, K/2]
  const void* act_scales;  // bf16 [M, K/64] | u8 [M, K/16]
  const float* lora_act;   // f32 [M, rank]
  const void* w_codes;     // u8 [N, K/2]
  const void* w_scales;    // bf16 [N, K/64] | u8 [N, K/16]
  const void* lora_up;     // bf16 [N, rank]
  const void* bias;        // bf16 [N] or null
  void* out;               // bf16 [M, N]
  int32_t* partials;       // parity export: i32 [M, N, K/G] (then out is unused)
  float wtscale;
  int64_t M, K, N;
  int precision, rank;
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

hipError_t launch_quantize_act(const QuantActArgs& a, hipStream_t stream);
hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream);
hipError_t launch_awq_gemv(const AwqArgs& a, hipStream_t stream);

}  // namespace svdq
