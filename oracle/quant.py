"""Group quantizers (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Every function works on a float32 matrix [rows, K] and quantizes each row in
contiguous groups of ``G`` columns, the group sizes of the "Supported
quantization types" table on the Nunchaku Lite pages (int4: 64, nvfp4: 16,
AWQ int4: 64).  All float arithmetic is IEEE float32 with round-to-nearest-even
(numpy float32 semantics), one rounding per written operation, because the GPU
must reproduce the same codes and scales bit for bit.

Readings (the pages name the formats only):

* int4 (symmetric): s = bf16(fl32(amax / 7)), q = rne(fl32(x * fl32(1/s))),
  |q| <= 7 always (s is at most 2^-8 below amax/7, so |x/s| < 7.03).
* nvfp4, activations: per-16 E4M3 scale s8 = E4M3(fl32(amax / 6)), tensor
  scale 1, S = dec(s8), code = E2M1(fl32(x * fl32(1/S))).
* nvfp4, weights: one fp32 tensor scale t = fl32(amax_tensor / 2688)
  (2688 = 6 * 448, so the largest block uses the whole E4M3 range);
  s8 = E4M3(fl32(amax / fl32(6 t))), S = fl32(dec(s8) * t),
  code = E2M1(fl32(x * fl32(1/S))).
* AWQ uint4 (asymmetric min-max round-to-nearest, range extended to 0):
  s = bf16(fl32((max - min) / 15)), z = clamp(rne(fl32(-min * fl32(1/s))), 0, 15),
  q = clamp(rne(fl32(x * fl32(1/s))) + z, 0, 15).
* Zero groups: amax (or max - min) below 2^-100, or a scale that rounds to 0,
  give scale 0 and all codes 0.
"""

import numpy as np

from .formats import (F32, bf16_round, bf16_bits, e4m3_encode, e4m3_decode,
                      e2m1_encode)

TINY = F32(2.0 ** -100)


def _groups(x, G):
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    if K % G:
        raise ValueError(f"K={K} is not a multiple of the group size {G}")
    return x.reshape(R, K // G, G)


def quantize_int4(x, G=64):
    """Symmetric int4 group quantizer.

    Returns (nibbles uint8 [R, K] sign-magnitude, scales float32 [R, K/G]
    holding bfloat16 values, q int64 [R, K] integer codes).
    """
    xg = _groups(x, G)
    amax = np.max(np.abs(xg), axis=2)
    zero = amax < TINY
    s = bf16_round(amax / F32(7.0))
    s = np.where(zero | (s == 0), F32(0.0), s).astype(F32)
    zero = s == 0
    inv = np.where(zero, F32(0.0), F32(1.0) / np.where(zero, F32(1.0), s)).astype(F32)
    t = (xg * inv[..., None]).astype(F32)
    mag = np.minimum(np.rint(np.abs(t)), 7).astype(np.int64)
    sign = np.signbit(t).astype(np.int64)
    nib = (mag | (sign << 3))
    nib = np.where(zero[..., None], 0, nib)
    q = np.where(sign == 1, -mag, mag)
    q = np.where(zero[..., None], 0, q)
    R, K = np.asarray(x).shape
    return nib.reshape(R, K).astype(np.uint8), s, q.reshape(R, K)


def quantize_nvfp4_act(x, G=16):
    """nvfp4 activation quantizer (tensor scale 1).

    Returns (E2M1 codes uint8 [R, K], E4M3 scale codes uint8 [R, K/G]).
    """
    xg = _groups(x, G)
    amax = np.max(np.abs(xg), axis=2)
    sf = (amax / F32(6.0)).astype(F32)
    s8 = e4m3_encode(sf)
    S = e4m3_decode(s8)
    zero = (amax < TINY) | (S == 0)
    s8 = np.where(zero, 0, s8).astype(np.uint8)
    inv = np.where(zero, F32(0.0), F32(1.0) / np.where(zero, F32(1.0), S)).astype(F32)
    t = (xg * inv[..., None]).astype(F32)
    codes = e2m1_encode(t)
    codes = np.where(zero[..., None], 0, codes)
    R, K = np.asarray(x).shape
    return codes.reshape(R, K).astype(np.uint8), s8


def quantize_nvfp4_weight(w, G=16):
    """nvfp4 weight quantizer with one fp32 tensor scale.

    Returns (E2M1 codes uint8 [N, K], E4M3 scale codes uint8 [N, K/G],
    tensor scale t as a Python float holding an fp32 value).
    """
    wg = _groups(w, G)
    amax_t = F32(np.max(np.abs(wg))) if wg.size else F32(0.0)
    if amax_t < TINY:
        N, K = np.asarray(w).shape
        return (np.zeros((N, K), np.uint8), np.zeros((N, K // G), np.uint8), 1.0)
    t = F32(amax_t / F32(2688.0))
    six_t = F32(F32(6.0) * t)
    amax = np.max(np.abs(wg), axis=2)
    sf = (amax / six_t).astype(F32)
    s8 = e4m3_encode(sf)
    S = (e4m3_decode(s8) * t).astype(F32)
    zero = (amax < TINY) | (S == 0)
    s8 = np.where(zero, 0, s8).astype(np.uint8)
    inv = np.where(zero, F32(0.0), F32(1.0) / np.where(zero, F32(1.0), S)).astype(F32)
    tq = (wg * inv[..., None]).astype(F32)
    codes = e2m1_encode(tq)
    codes = np.where(zero[..., None], 0, codes)
    N, K = np.asarray(w).shape
    return codes.reshape(N, K).astype(np.uint8), s8, float(t)


def quantize_awq(w, G=64):
    """AWQ-style asymmetric uint4 group quantizer.

    Returns (q uint8 [N, K] in 0..15, scales float32 [N, K/G] holding bf16
    values, zeros float32 [N, K/G] holding integers 0..15).
    """
    wg = _groups(w, G)
    wmin = np.minimum(np.min(wg, axis=2), F32(0.0)).astype(F32)
    wmax = np.maximum(np.max(wg, axis=2), F32(0.0)).astype(F32)
    rng = (wmax - wmin).astype(F32)
    s = bf16_round((rng / F32(15.0)).astype(F32))
    zero = (rng < TINY) | (s == 0)
    s = np.where(zero, F32(0.0), s).astype(F32)
    inv = np.where(zero, F32(0.0), F32(1.0) / np.where(zero, F32(1.0), s)).astype(F32)
    z = np.clip(np.rint((-wmin * inv).astype(F32)), 0, 15)
    q = np.clip(np.rint((wg * inv[..., None]).astype(F32)) + z[..., None], 0, 15)
    q = np.where(zero[..., None], 0, q)
    z = np.where(zero, 0, z)
    N, K = np.asarray(w).shape
    return q.reshape(N, K).astype(np.uint8), s, z.astype(F32)


def dequant_int4(q, s, G=64):
    """Integer codes [R, K] and group scales [R, K/G] -> float64 values."""
    q = np.asarray(q, dtype=np.float64)
    R, K = q.shape
    return (q.reshape(R, K // G, G) * np.asarray(s, np.float64)[..., None]).reshape(R, K)


def scales_bits(s):
    """float32 bf16-valued scales -> uint16 bit patterns (exact)."""
    b = bf16_bits(s)
    return b
