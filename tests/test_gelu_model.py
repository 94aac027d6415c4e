"""A CPU model of the fused MLP epilogue's GELU evaluation, checked against
the oracle's bf16 GELU on every bf16 input.

The epilogue evaluates GELU with the exact erf in float32 as
(y/2) erfc(-y / sqrt 2), with erfc(-a) = 2 - erfc(a) for y > 0 and erfc from
the Chebyshev fit of Numerical Recipes in C (2nd ed., section 6.2, "erfcc":
t = 1 / (1 + z/2), erfc(z) = t exp(-z^2 + P(t)), fractional error < 1.2e-7).
The model below performs the same float32 operations (each fused
multiply-add rounded once; reciprocal and exp exact, then rounded) and must
round to the same bf16 as gelu_bf16 wherever the GELU is a normal number:
the fit's error stays below half a bf16 ulp there.  The kernel's own hardware
reciprocal and exp are checked by the GPU parity tests of the fused MLP.
"""

import numpy as np

from oracle import formats as F, layers as L

f32 = np.float32

# P(t) of the fit, highest degree first
_P = (0.17087277, -0.82215223, 1.48851587, -1.13520398, 0.27886807, -0.18628806, 0.09678418, 0.37409196,
      1.00002368, -1.26551223)


def _fma32(a, b, c):
    # a*b of two float32 values is exact in float64; one rounding of the sum
    # to float64 and then float32 (double rounding is possible but rare)
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(f32)


def _gelu_model(y):
    y = y.astype(f32)
    z = (np.abs(y) * f32(0.70710678118654752)).astype(f32)
    t = (1.0 / _fma32(np.full_like(z, 0.5), z, np.ones_like(z)).astype(np.float64)).astype(f32)
    q = np.full_like(t, f32(_P[0]))
    for c in _P[1:]:
        q = _fma32(t, q, np.full_like(t, f32(c)))
    with np.errstate(under="ignore", over="ignore"):
        e = (t * np.exp(_fma32(-z, z, q).astype(np.float64)).astype(f32)).astype(f32)
    half = (y * f32(0.5)).astype(f32)
    return (half * np.where(y > 0, (f32(2.0) - e).astype(f32), e)).astype(f32)


def test_gelu_model_rounds_like_the_oracle_on_every_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    y = F.bf16_to_f32(bits)
    fin = np.isfinite(y)
    bits, y = bits[fin], y[fin]
    ref = L.gelu_bf16(bits)
    got = F.bf16_bits_f64(_gelu_model(y).astype(np.float64))
    ref_v = np.abs(F.bf16_to_f32(ref).astype(np.float64))
    normal = ref_v >= 2.0 ** -126
    assert normal.sum() > 45000
    bad = np.nonzero((got != ref) & normal)[0]
    assert bad.size == 0, [(float(y[i]), int(got[i]), int(ref[i])) for i in bad[:8]]
    # zeros and subnormal results: the model's value is within one bf16
    # quantum (2^-133) of the correctly rounded one
    sub = ~normal
    diff = np.abs(F.bf16_to_f32(got[sub]).astype(np.float64) - F.bf16_to_f32(ref[sub]).astype(np.float64))
    assert np.all(diff <= 2.0 ** -133)


def test_gelu_model_fit_error():
    # relative error of the float32 model for y in [-14, 0), where erfc's
    # argument spans (0, 9.9], wherever erfc itself is a normal float32
    y = -np.linspace(0.0, 14.0, 20001)[1:].astype(f32)
    model = _gelu_model(y).astype(np.float64)
    exact = L.gelu_f64(y.astype(np.float64))
    ok = np.abs(exact / (0.5 * y.astype(np.float64))) >= 2.0 ** -126
    assert ok.sum() > 18000
    rel = np.abs(model[ok] - exact[ok]) / np.abs(exact[ok])
    # the fit's own 1.2e-7 plus float32 rounding; the rounding of z = |y|/sqrt 2
    # (relative 2^-24) moves exp(-z^2) by up to 2 z^2 2^-24 = 1.2e-5 at z = 9.3;
    # all far below half a bf16 ulp (2^-9)
    assert rel[np.abs(y[ok]) <= 2.0].max() < 1.0e-6
    assert rel.max() < 2.0e-5
