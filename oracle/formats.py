"""Bit-level number formats used by the quantized linears (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Formats
-------
* bfloat16 -- the pages' ``compute_dtype`` ("NunchakuLiteQuantizationConfig"
  section: floating-point buffers of quantized modules are bfloat16).  Stored
  here as uint16 bit patterns; rounding is IEEE round-to-nearest-even.
* OCP E4M3 (``float8_e4m3fn``) -- the nvfp4 block-scale format.  Reading: bias 7,
  subnormals m*2^-9, largest finite 448, no infinities; encoding rounds to
  nearest even and saturates to +-448 ("satfinite").
* OCP E2M1 -- the nvfp4 element format ("Supported quantization types" table,
  precision ``nvfp4``).  Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; encoding rounds
  to nearest even and saturates to +-6.  The sign bit (bit 3) is the sign bit
  of the encoded fp32 value, so -0.0 and small negatives encode as 0x8.
* int4 codes (precision ``int4``).  Reading: *sign-magnitude* nibbles, bit 3 =
  sign, bits 0..2 = |q| in 0..7.  The symmetric quantizer (scale = amax/7)
  never produces |q| > 7, so the two's-complement-only value -8 is not needed.
  Same sign convention as E2M1.
* AWQ uint4 codes: plain unsigned nibbles 0..15.
* Nibble packing (both precisions): row-major [rows, K/2] bytes, the low
  nibble of byte j holds element 2j, the high nibble element 2j+1.
"""

import numpy as np

F32 = np.float32


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------
def bf16_bits(x):
    """Round float32 values to bfloat16 (RNE); return the uint16 bit patterns."""
    x = np.asarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_to_f32(b):
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(F32)


def bf16_round(x):
    """float32 -> nearest bfloat16 value, returned as float32 (RNE)."""
    return bf16_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------
# OCP E4M3 (float8_e4m3fn)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(b):
    """uint8 E4M3 codes -> float32 values (0x7F/0xFF decode as NaN)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(F32)


def e4m3_encode(v):
    """float32 -> uint8 E4M3 code: round to nearest even on the E4M3 grid,
    saturating to +-448.  Inputs must be finite.

    Written from the format definition: in the binade [2^e, 2^(e+1)) with
    e >= -6 the grid step is 2^(e-3); below 2^-6 (subnormals) the step is 2^-9.
    The value is scaled by the step (exact in fp64), rounded half-to-even with
    ``np.rint``, and the rounded magnitude is re-encoded as exponent/mantissa.
    """
    v = np.asarray(v, dtype=F32).astype(np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.int64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # guard against log2 rounding at binade edges
    e = np.where(np.power(2.0, e) > a, e - 1, e)
    e = np.where(np.power(2.0, e + 1) <= a, e + 1, e)
    e = np.maximum(e, -6.0)
    step = np.power(2.0, e - 3)
    r = np.rint(a / step) * step
    r = np.minimum(r, E4M3_MAX)
    # re-encode r (a grid value, possibly carried into the next binade)
    out = np.zeros(v.shape, dtype=np.int64)
    sub = r < 2.0 ** -6
    out = np.where(sub, np.rint(r / 2.0 ** -9).astype(np.int64), out)
    with np.errstate(divide="ignore"):
        er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    er = np.where(np.power(2.0, er) > r, er - 1, er)
    mant = np.rint((r / np.power(2.0, er) - 1.0) * 8).astype(np.int64)
    normal_code = ((er.astype(np.int64) + 7) << 3) | mant
    out = np.where(sub, out, normal_code)
    return (out | (sign << 7)).astype(np.uint8)


# ----------------------------------------------------------------------------
# OCP E2M1
# ----------------------------------------------------------------------------
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(n):
    """4-bit E2M1 codes (0..15) -> float32 values."""
    n = np.asarray(n).astype(np.int64)
    mag = E2M1_GRID[n & 7]
    return np.where((n & 8) != 0, -mag, mag).astype(F32)


def e2m1_encode(v):
    """float32 -> 4-bit E2M1 code (0..15), RNE on the E2M1 grid, saturating at 6.

    From the format definition: the grid step is 0.5 below 2, 1 on [2, 4) and
    2 from 4 upward; scaling by the step is exact, ``np.rint`` rounds half to
    even (an even multiple of the step is an even mantissa code), and results
    above 6 saturate.  Sign bit = IEEE sign bit of ``v``.
    """
    v = np.asarray(v, dtype=F32).astype(np.float64)
    a = np.abs(v)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / step) * step, 6.0)
    mag_code = np.searchsorted(E2M1_GRID, r)  # r is exactly a grid value
    return (mag_code | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


# ----------------------------------------------------------------------------
# int4 sign-magnitude codes
# ----------------------------------------------------------------------------
def int4_to_nibble(q):
    """Integer codes in [-7, 7] -> sign-magnitude nibbles (bit 3 = sign)."""
    q = np.asarray(q).astype(np.int64)
    if np.any(np.abs(q) > 7):
        raise ValueError("int4 codes must lie in [-7, 7]")
    return ((np.abs(q) & 7) | ((q < 0).astype(np.int64) << 3)).astype(np.uint8)


def nibble_to_int4(n):
    """Sign-magnitude nibbles -> integer codes in [-7, 7] (0x8 decodes to 0)."""
    n = np.asarray(n).astype(np.int64)
    mag = n & 7
    return np.where((n & 8) != 0, -mag, mag)


# ----------------------------------------------------------------------------
# nibble packing
# ----------------------------------------------------------------------------
def pack_nibbles(codes):
    """[rows, K] codes in 0..15 -> [rows, K/2] uint8, low nibble = even k."""
    c = np.asarray(codes).astype(np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even")
    if np.any(c > 15):
        raise ValueError("codes must fit in 4 bits")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[rows, K/2] uint8 -> [rows, K] codes in 0..15."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def bf16_bits_f64(x):
    """float64 -> bfloat16 bits with a single round-to-nearest-even step.

    Values start in float64 (weight preparation, the GELU reference).  A
    normal value is written as m * 2^e with 0.5 <= |m| < 1 and m rounded to 8
    significant bits with ``np.rint`` (exact scaling by 256); below the
    normal range (|x| < 2^-126) bfloat16 has the fixed quantum 2^-133 of its
    subnormals, and x / 2^-133 is rounded with ``np.rint``.  The result is
    exactly representable in float32 and bfloat16 and is re-encoded.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0), e - 8)
    sub = np.abs(x) < 2.0 ** -126
    r = np.where(sub, np.rint(x * 2.0 ** 133) * 2.0 ** -133, r)
    r = np.where(r == 0, np.copysign(0.0, x), r)
    return bf16_bits(r.astype(F32))


# ----------------------------------------------------------------------------
# IEEE binary16 (the matrix-instruction operand format of the GPU path)
# ----------------------------------------------------------------------------
F16_MAX = 65504.0


def f16_round(x):
    """float64 -> the nearest IEEE binary16 value (round half to even),
    returned as float64.  Finite inputs with |x| below 65520 (the rounding
    boundary of the largest finite value) only.

    From the format definition: 11 significant bits for normal values
    (|x| >= 2^-14), written as m * 2^e with 0.5 <= |m| < 1 and m scaled by
    2^11 (exact) and rounded with ``np.rint``; below 2^-14 the fixed quantum
    of the subnormals, 2^-24.  The sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) >= 65520.0):
        raise ValueError("f16_round: input outside the finite binary16 range")
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 2048.0), e - 11)
    sub = np.abs(x) < 2.0 ** -14
    r = np.where(sub, np.rint(x * 2.0 ** 24) * 2.0 ** -24, r)
    return np.where(r == 0, np.copysign(0.0, x), r)
