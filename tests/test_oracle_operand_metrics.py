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


def test_operand_int4_codes_as_e4m3():
    # every nibble: the E4M3 byte torch's float8_e4m3fn cast gives for the
    # signed integer (the code 0x8 is -0, byte 0x80), and the byte decodes back
    # to the integer
    torch = pytest.importorskip("torch")
    nib = np.tile(np.arange(16, dtype=np.uint8), 4)[None, :]  # [1, 64]: one int4 group
    q8, sc = L.product_operand_ref(nib, F.bf16_bits(np.array([[0.5]], np.float32)), "int4")
    mag = (nib & 7).astype(np.float32)
    signed = np.where(nib & 8, -mag, mag)
    want = torch.from_numpy(signed).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert q8.dtype == np.uint8 and np.array_equal(q8, want)
    assert np.array_equal(q8[0, :16], [0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E,
                                       0x80, 0xB8, 0xC0, 0xC4, 0xC8, 0xCA, 0xCC, 0xCE])
    assert np.array_equal(F.e4m3_decode(q8).astype(np.float64), signed.astype(np.float64))
    assert np.array_equal(np.signbit(F.e4m3_decode(q8)), np.signbit(signed))
    assert sc.shape == (1, 1) and sc[0, 0] == 0.5


def test_operand_int4_reassembles_the_dequantization():
    # codes times group scales give back dequant() for rows of every scale
    # magnitude (no window: the scales stay separate)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((12, 512)).astype(np.float32)
    x[1] *= 3e5
    x[2] *= 1e-7
    x[3, 256:] *= 1e-9
    x[4] = 0.0
    x[5, 64:] = 0.0
    x[6, :64] *= 1e20
    nib, s, q = quantize_int4(F.bf16_round(x), 64)
    q8, sc = L.product_operand_ref(nib, F.bf16_bits(s), "int4")
    deq = L.dequant(nib, F.bf16_bits(s), "int4")
    vals = F.e4m3_decode(q8).astype(np.float64).reshape(12, 8, 64) * sc[..., None]
    assert np.array_equal(vals.reshape(12, 512), deq)
    assert np.array_equal(sc, s.astype(np.float64))


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
