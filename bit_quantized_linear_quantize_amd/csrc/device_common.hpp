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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
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

// float64 -> bf16 bits, one round-to-nearest-even step (bf16 subnormals have
// the quantum 2^-133; overflow gives infinity)
__device__ __forceinline__ uint16_t bf16_from_f64(double v) {
  const double a = fabs(v);
  double r;
  if (a < 0x1p-126) {
    r = rint(v * 0x1p133) * 0x1p-133;
  } else {
    // keep 7 of the 52 fraction bits: add half an ulp minus one plus the
    // kept lowest bit (ties to even), then clear the 45 dropped bits
    uint64_t u = (uint64_t)__double_as_longlong(v);
    u += 0xFFFFFFFFFFFull + ((u >> 45) & 1ull);
    u &= ~0x1FFFFFFFFFFFull;
    r = __longlong_as_double((long long)u);
  }
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// Two floats -> packed bf16 pair (RNE), low half = a, with the hardware
// pair conversion (finite inputs).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Two floats -> packed bf16 pair (RNE), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// Raw buffer descriptor over `bytes` bytes at p (sizes past 2^31 - 1 are
// clamped: a tile never addresses that far from its base).  Loads at offsets
// at or past `bytes` return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, size_t bytes) {
  const int n = bytes > 0x7fffffffu ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
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

// Eight sign-magnitude int4 codes (nibble i = bits 4i..4i+3 = column i, bit 3
// = sign, bits 0..2 = |q| <= 7) -> eight fp16 values q in column order, as
// four (column 2i, column 2i+1) pairs.  Each |q| is looked up with v_perm in
// the table of the high bytes of the fp16 encodings of 0..7 (their low bytes
// are 0); the sign bit moves to bit 7 of the high byte.  Exact.
__device__ __forceinline__ u32x4 int4x8_to_f16(uint32_t w) {
  constexpr uint32_t kT0 = 0x42403C00u;  // fp16 high bytes of 0, 1, 2, 3
  constexpr uint32_t kT1 = 0x47464544u;  // of 4, 5, 6, 7
  const uint32_t mlo = w & 0x07070707u;          // |q| of columns 0, 2, 4, 6
  const uint32_t mhi = (w >> 4) & 0x07070707u;   // |q| of columns 1, 3, 5, 7
  const uint32_t hlo = __builtin_amdgcn_perm(kT1, kT0, mlo) | ((w << 4) & 0x80808080u);
  const uint32_t hhi = __builtin_amdgcn_perm(kT1, kT0, mhi) | (w & 0x80808080u);
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(hhi, hlo, 0x040C000Cu);  // (q0, q1)
  r[1] = __builtin_amdgcn_perm(hhi, hlo, 0x050C010Cu);  // (q2, q3)
  r[2] = __builtin_amdgcn_perm(hhi, hlo, 0x060C020Cu);  // (q4, q5)
  r[3] = __builtin_amdgcn_perm(hhi, hlo, 0x070C030Cu);  // (q6, q7)
  return r;
}

// The same codes times an fp16 scale (exact whenever q * scale is an fp16).
__device__ __forceinline__ f16x8 int4x8_to_f16_scaled(uint32_t w, _Float16 scale) {
  const f16x8 v = __builtin_bit_cast(f16x8, int4x8_to_f16(w));
  const f16x8 sc = {scale, scale, scale, scale, scale, scale, scale, scale};
  return v * sc;
}

// Eight OCP E2M1 codes (nibble i = column i) times an fp16 scale -> fp16 in
// column order.  E2M1 -> fp16 is exact (scale operand 1: the conversion
// applies only a power of two); exact whenever value * scale is an fp16.
__device__ __forceinline__ f16x8 e2m1x8_to_f16_scaled(uint32_t w, _Float16 scale) {
  const f16x2 sc = {scale, scale};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// nvfp4 activation quantizer for one group of 16 values x[0..15]: per-token
// block scale s8 = E4M3(fl32(amax / 6)) (tensor scale 1; round to nearest
// even, saturating at 448), codes = E2M1(fl32(x * fl32(1 / dec(s8)))) with
// nibble i = value i; a group with amax < 2^-100 or dec(s8) == 0 gets codes
// 0.  Returns the E4M3 byte (0 for such a group) and dec(s8) in S.
__device__ __forceinline__ uint32_t nvfp4_quant16(const float* x, uint32_t& cw0, uint32_t& cw1, float& S) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float sf = __fdiv_rn(amax, 6.0f);
  const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(sf, 448.0f), 0.0f, 0, false) & 0xffu;
  S = __builtin_amdgcn_cvt_f32_fp8((int)s8, 0);
  const bool zero = !(amax >= kTiny) || S == 0.0f;
  const float inv = zero ? 0.f : __fdiv_rn(1.0f, S);
  cw0 = 0;
  cw1 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t0 = __fmul_rn(x[2 * j], inv);
    const float t1 = __fmul_rn(x[2 * j + 1], inv);
    const uint32_t byte = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t0, t1, 1.0f, 0) & 0xffu;
    if (j < 4) cw0 |= byte << (8 * j);
    else cw1 |= byte << (8 * (j - 4));
  }
  cw0 = zero ? 0u : cw0;
  cw1 = zero ? 0u : cw1;
  return zero ? 0u : s8;
}

}  // namespace svdq
