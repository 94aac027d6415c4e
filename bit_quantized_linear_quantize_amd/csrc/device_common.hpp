// Device-side helpers shared by the gfx950 kernels.
//
// Register layouts of the matrix instructions used here (wave64; checked on
// gfx950 against host matrix products):
//   32x32xK (bf16 K=16, f16 K=16, fp8 scaled K=64):
//     A operand: lane l holds row l%32, k-slots (l/32, i);
//     B operand: lane l holds column l%32, k-slots (l/32, i) -- the same slot
//     function as A, so any consistent assignment of real k to slots is a
//     valid contraction;
//     D: lane l, register j holds row (j/4)*8 + (l/32)*4 + j%4, column l%32.
//   16x16x32 bf16:
//     A: lane l holds row l%16, slots (l/16, i); B likewise with column l%16;
//     D: lane l, register j holds row (l/16)*4 + j, column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace svdq {

constexpr float kTiny = 7.888609052210118e-31f;  // 2^-100: zero-group threshold

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// IEEE float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> packed bf16 pair (RNE), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for the
// wave's outstanding global loads (its release fence covers global memory),
// which would stall a software pipeline whose prefetches are still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// Sign-magnitude nibbles -> OCP E4M3 bytes.  Magnitude codes 0..7 map to the
// E4M3 encodings of the values given by `lut_lo` (codes 0..3) and `lut_hi`
// (codes 4..7); bit 3 of a nibble becomes bit 7 of its byte.  For the eight
// nibbles of `w` (nibble i = bits 4i..4i+3) the results are returned as
//   lo = bytes for nibbles 0, 2, 4, 6 and hi = bytes for nibbles 1, 3, 5, 7.
// (Any fixed order of k inside a group is a valid contraction as long as both
// operands use the same one.)
__device__ __forceinline__ void nibbles_to_e4m3(uint32_t w, uint32_t lut_lo, uint32_t lut_hi,
                                                uint32_t& lo, uint32_t& hi) {
  uint32_t sel_lo = w & 0x07070707u;
  uint32_t sel_hi = (w >> 4) & 0x07070707u;
  lo = __builtin_amdgcn_perm(lut_hi, lut_lo, sel_lo) | ((w << 4) & 0x80808080u);
  hi = __builtin_amdgcn_perm(lut_hi, lut_lo, sel_hi) | (w & 0x80808080u);
}

// E4M3 encodings of the int4 magnitudes 0..7 and of the E2M1 magnitudes
// 0, .5, 1, 1.5, 2, 3, 4, 6 (as 4-byte lookup tables for v_perm_b32).
constexpr uint32_t kInt4LutLo = 0x44403800u;   // 0, 1, 2, 3
constexpr uint32_t kInt4LutHi = 0x4E4C4A48u;   // 4, 5, 6, 7
constexpr uint32_t kE2m1LutLo = 0x3C383000u;   // 0, .5, 1, 1.5
constexpr uint32_t kE2m1LutHi = 0x4C484440u;   // 2, 3, 4, 6

}  // namespace svdq
