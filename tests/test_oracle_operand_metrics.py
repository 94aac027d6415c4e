"""Pins (CPU) of the oracle's binary16 rounding, its reference for the product
operand the linear's first kernel writes, and the error metrics every output
test uses (bf16_half_ulp, output_errors).

Each check is tied to something other than the function itself: brute force
over every value of the format, numpy's float16 cast (a library routine),
closed forms, and plain Python loops with math.fsum."""

import math

import numpy as np
import pytest

from oracle import formats as F, layers as L
from oracle.quant import quantize_int4, quantize_nvfp4_act

# every finite positive binary16 / bfloat16 value, ascending
F16_POS = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
BF16_POS = F.bf16_to_f32(np.arange(0, 0x7F80, dtype=np.uint16)).astype(np.float64)


def nearest_even_brute(x, grid, codes_even):
    """RNE onto `grid` (ascending non-negative values) by brute force: the
    nearest grid value, ties to the one whose code is even."""
    a = abs(x)
    d = np.abs(grid - a)
    best = np.flatnonzero(d == d.min())
    if len(best) > 1:
        best = [b for b in best if codes_even[b]]
    return math.copysign(grid[best[0]], x)


# ------------------------------------------------------------------ f16_round
def test_f16_round_brute_force_with_midpoints():
    rng = np.random.default_rng(0)
    mids = (F16_POS[1:] + F16_POS[:-1]) / 2
    pick = rng.choice(len(mids), 3000, replace=False)
    xs = np.concatenate([mids[pick], F16_POS[pick], rng.uniform(0, 65504, 500),
                         np.exp2(rng.uniform(-26, 15.9, 2000)), [0.0, 2.0 ** -25, 3 * 2.0 ** -26, 65504.0, 65519.0]])
    xs = np.concatenate([xs, -xs])
    even = (np.arange(len(F16_POS)) % 2) == 0
    got = F.f16_round(xs)
    for x, g in zip(xs, got):
        assert g == nearest_even_brute(x, F16_POS, even), x


def test_f16_round_matches_numpy_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-28, 15, 200000))
    x = x[np.abs(x) < 65504]
    assert np.array_equal(F.f16_round(x), x.astype(np.float16).astype(np.float64))
    assert np.signbit(F.f16_round(np.array([-1e-30])))[0]
    with pytest.raises(ValueError):
        F.f16_round(np.array([65520.0]))


# ------------------------------------------------------------------ product operand
def f16_exact(v):
    return np.array_equal(F.f16_round(v), v)


def test_operand_nvfp4_is_the_exact_dequantization():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((40, 256)) * np.exp2(rng.integers(-12, 8, (40, 1)))).astype(np.float32)
    codes, scales = quantize_nvfp4_act(x, 16)
    vals, rs = L.product_operand_ref(codes, scales, "nvfp4")
    assert rs is None
    assert np.array_equal(vals, L.dequant(codes, scales, "nvfp4"))
    assert f16_exact(vals)


def brute_exponent(scales_row):
    """E by search: 0 if every nonzero scale lies in [2^-17, 2^13), else the
    E with max(scale) * 2^-E in [2^12, 2^13)."""
    nz = scales_row[scales_row > 0]
    if nz.size == 0 or (nz.max() < 2.0 ** 13 and nz.min() >= 2.0 ** -17):
        return 0
    for E in range(-300, 300):
        if 2.0 ** 12 <= nz.max() * 2.0 ** -E < 2.0 ** 13:
            return E
    raise AssertionError


def int4_rows():
    rng = np.random.default_rng(3)
    K = 512
    x = rng.standard_normal((12, K)).astype(np.float32)
    x[1] *= 3e5                                   # all scales above 2^13
    x[2] *= 1e-7                                  # all below 2^-17
    x[3, 256:] *= 1e-9                            # spread 2^-33 .. 2^-1: beyond 2^29, rounded
    x[4] = np.clip(x[4], -3, 3)
    x[4, 5] = 57088.0                             # s = 8160: fits
    x[5] = np.clip(x[5], -3, 3)
    x[5, 70] = 57344.0                            # s = 8192: rewritten
    x[6, 128:192] *= 1e-9
    x[6, 130] = 7 * 2.0 ** -17                    # smallest s = 2^-17: fits
    x[7, 128:192] *= 1e-9
    x[7, 130] = 1.734375 * 2.0 ** -15             # just below 2^-17: rewritten
    x[8] = 0.0                                    # zero row
    x[9, 64:] = 0.0
    x[10, :64] *= 1e20                            # one huge group, the rest far below 2^29 of it
    x = F.bf16_round(x)
    return quantize_int4(x, 64)


def test_operand_int4_row_exponents_by_search():
    nib, s, q = int4_rows()
    vals, rs = L.product_operand_ref(nib, F.bf16_bits(s), "int4")
    deq = L.dequant(nib, F.bf16_bits(s), "int4")
    for m in range(nib.shape[0]):
        E = brute_exponent(s[m].astype(np.float64))
        assert rs[m] == 2.0 ** E, m
        assert f16_exact(vals[m])
        sm = s[m].astype(np.float64)
        near = np.repeat(sm >= sm.max() * 2.0 ** -29, 64)
        # groups within 2^29 of the largest scale: exact (values * 2^E is the dequantization)
        assert np.array_equal(vals[m][near] * 2.0 ** E, deq[m][near]), m
        # below that: two roundings to binary16 (the scale, then the product),
        # each at most half a binary16 subnormal quantum 2^-25 (relative 2^-11 above it)
        far = ~near
        if far.any():
            err = np.abs(vals[m][far] * 2.0 ** E - deq[m][far])
            bound = (7 * 2.0 ** -25 + 2.0 ** -25 + 2.0 ** -11 * np.abs(deq[m][far]) * 2.0 ** -E) * 2.0 ** E
            assert np.all(err <= bound), m
    assert [brute_exponent(s[m].astype(np.float64)) != 0 for m in (4, 5, 6, 7)] == [False, True, False, True]


# ------------------------------------------------------------------ bf16_half_ulp
def brute_half_ulp(y):
    """Half the gap between the bfloat16 value at or below |y| and the next."""
    a = abs(y)
    i = np.searchsorted(BF16_POS, a, side="right") - 1
    return (BF16_POS[i + 1] - BF16_POS[i]) / 2


def test_bf16_half_ulp_brute_force():
    rng = np.random.default_rng(4)
    pows = np.exp2(np.arange(-140, 127, dtype=np.float64))
    ys = np.concatenate([pows, np.nextafter(pows, 0), np.nextafter(pows, np.inf), -pows,
                         rng.standard_normal(3000) * np.exp2(rng.integers(-130, 120, 3000)),
                         [0.0, 2.0 ** -133, 2.0 ** -126, np.nextafter(2.0 ** -126, 0)]])
    got = L.bf16_half_ulp(ys)
    for y, g in zip(ys, got):
        assert g == brute_half_ulp(y), y


def test_bf16_half_ulp_bounds_the_rounding_error():
    # RNE to bfloat16 never moves a value by more than the half-ulp, and
    # exact midpoints move by exactly that much
    rng = np.random.default_rng(5)
    y = rng.standard_normal(100000) * np.exp2(rng.integers(-120, 120, 100000))
    r = F.bf16_to_f32(F.bf16_bits_f64(y)).astype(np.float64)
    assert np.all(np.abs(r - y) <= L.bf16_half_ulp(y))
    mid = (BF16_POS[1000:1100] + BF16_POS[1001:1101]) / 2
    rm = F.bf16_to_f32(F.bf16_bits_f64(mid)).astype(np.float64)
    assert np.array_equal(np.abs(rm - mid), L.bf16_half_ulp(mid))


# ------------------------------------------------------------------ output_errors
def brute_errors(g, r):
    g, r = [float(v) for v in g.ravel()], [float(v) for v in r.ravel()]
    err = [abs(a - b) for a, b in zip(g, r)]
    rms = math.sqrt(math.fsum(v * v for v in r) / len(r))
    excess = max(e - brute_half_ulp(b) for e, b in zip(err, r))
    mre = math.fsum(err) / math.fsum(abs(v) for v in r)
    return max(err) / rms, excess / rms, mre


def test_output_errors_brute_force():
    rng = np.random.default_rng(6)
    for shape in [(3, 5), (8, 16), (1, 7)]:
        r = rng.standard_normal(shape) * 3
        g = F.bf16_to_f32(F.bf16_bits_f64(r + rng.standard_normal(shape) * 1e-3)).astype(np.float64)
        got = L.output_errors(g, r)
        want = brute_errors(g, r)
        assert np.allclose(got, want, rtol=1e-12, atol=0), (got, want)


def test_output_errors_closed_forms():
    r = np.ones((4, 4))
    g = r.copy()
    g[2, 3] += 0.5
    maxrel, excess, mre = L.output_errors(g, r)
    assert maxrel == 0.5                        # RMS(r) = 1
    assert excess == 0.5 - 2.0 ** -8            # half a bf16 ulp of 1.0 is 2^-8
    assert mre == 0.5 / 16
    # exact agreement
    assert L.output_errors(r, r)[0] == 0.0 and L.output_errors(r, r)[2] == 0.0
