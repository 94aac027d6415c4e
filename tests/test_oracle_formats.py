"""Pins for oracle/formats.py: brute force over each format's grid and the
library casts of torch (bfloat16, float8_e4m3fn)."""

import struct

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import formats as F


def _f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


# ---------------------------------------------------------------- bfloat16
def _sweep_f32(n=200000, seed=0):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # exact bf16 midpoints and their neighbours
    base = rng.integers(0, 2 ** 16, size=5000, dtype=np.uint32) << 16
    mid = (base | 0x8000).view(np.float32)
    with np.errstate(invalid='ignore'):
        near = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))])
    near = near[np.isfinite(near)]
    return np.concatenate([x, near]).astype(np.float32)


def test_bf16_matches_torch_cast():
    x = _sweep_f32()
    ours = F.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_roundtrip_exact():
    b = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(b)
    ok = np.isfinite(v)
    assert np.array_equal(F.bf16_bits(v[ok]), b[ok])


def test_bf16_from_f64_single_rounding_brute_force():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000),
                        # exact ties between bf16 neighbours, in float64
                        (np.arange(1, 2000) * 2 + 1) * 2.0 ** -9 + 1.0])
    got = F.bf16_to_f32(F.bf16_bits_f64(x)).astype(np.float64)
    for xi, gi in zip(x[:4000], got[:4000]):
        # neighbours of xi on the bf16 grid by brute force over the exponent
        m, e = np.frexp(xi)
        lo = np.floor(m * 256) * 2.0 ** (e - 8)
        hi = lo + 2.0 ** (e - 8)
        dl, dh = abs(xi - lo), abs(hi - xi)
        if dl < dh:
            want = lo
        elif dh < dl:
            want = hi
        else:  # tie: even last mantissa bit
            want = lo if int(round(abs(lo) / 2.0 ** (e - 8))) % 2 == 0 else hi
        assert gi == want, (xi, gi, want)
    # the tie set: 1 + odd * 2^-9 lies halfway between bf16 neighbours
    ties = x[20000:]
    g = F.bf16_to_f32(F.bf16_bits_f64(ties)).astype(np.float64)
    k = np.rint((g - 1.0) / 2.0 ** -8).astype(np.int64)
    assert np.all(k % 2 == 0)


def test_bf16_from_f64_subnormals():
    # below 2^-126 the bf16 grid has the fixed quantum 2^-133: values that are
    # exactly float32 take the float32 route's rounding (bf16_bits, integer
    # rounding of the bit pattern), and exact halfway points go to even
    rng = np.random.default_rng(2)
    x32 = (rng.integers(1, 2 ** 23, 5000).astype(np.uint32)).view(np.float32)  # float32 subnormals
    x32 = np.concatenate([x32, -x32])
    assert np.array_equal(F.bf16_bits_f64(x32.astype(np.float64)), F.bf16_bits(x32))
    q = 2.0 ** -133
    ties = (np.arange(1, 200) * 2 + 1) * q / 2   # halfway between k q and (k + 1) q
    k = np.rint(F.bf16_to_f32(F.bf16_bits_f64(ties)).astype(np.float64) / q).astype(np.int64)
    assert np.all(k % 2 == 0)
    assert F.bf16_bits_f64(np.array([q / 4]))[0] == 0 and F.bf16_bits_f64(np.array([-q / 4]))[0] == 0x8000


# ---------------------------------------------------------------- E4M3
ALL_E4M3 = np.arange(256, dtype=np.uint32).astype(np.uint8)


def test_e4m3_decode_matches_torch():
    ours = F.e4m3_decode(ALL_E4M3)
    ref = torch.from_numpy(ALL_E4M3.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _e4m3_brute(v):
    """Nearest finite E4M3 code by exhaustive search; ties -> even mantissa; saturate."""
    vals = F.e4m3_decode(ALL_E4M3).astype(np.float64)
    finite = ~np.isnan(vals)
    out = []
    for x in np.asarray(v, np.float64):
        if abs(x) > 448:
            out.append(0x7E if x > 0 else 0xFE)
            continue
        cand = [c for c in range(256) if finite[c] and (np.signbit(vals[c]) == np.signbit(x))]
        d = np.array([abs(vals[c] - x) for c in cand])
        best = [cand[i] for i in np.flatnonzero(d == d.min())]
        even = [c for c in best if c % 2 == 0]
        out.append((even or best)[0])
    return np.array(out, dtype=np.uint8)


def _e4m3_sweep():
    vals = F.e4m3_decode(ALL_E4M3).astype(np.float64)
    vals = vals[~np.isnan(vals)]
    pos = np.unique(np.abs(vals))
    mids = (pos[1:] + pos[:-1]) / 2
    pts = np.concatenate([pos, mids, [450.0, 463.0, 464.0, 465.0, 1e4, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]])
    pts32 = pts.astype(np.float32)
    pts32 = np.concatenate([pts32, np.nextafter(pts32, np.float32(np.inf)), np.nextafter(pts32, np.float32(0))])
    return np.concatenate([pts32, -pts32]).astype(np.float32)


def test_e4m3_encode_brute_force():
    v = _e4m3_sweep()
    assert np.array_equal(F.e4m3_encode(v), _e4m3_brute(v))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    v = np.concatenate([_e4m3_sweep(), (rng.standard_normal(50000) * 50).astype(np.float32)])
    v = v[np.abs(v) <= 448].astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_encode(v)
    # torch keeps the sign of values that round to zero; so do we
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    assert F.e4m3_encode(np.float32([500.0, 1e30, -1e9]))[0] == 0x7E
    assert list(F.e4m3_encode(np.float32([500.0, 1e30, -1e9]))) == [0x7E, 0x7E, 0xFE]


# ---------------------------------------------------------------- E2M1
def _e2m1_brute(x):
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = abs(float(x))
    if a > 6:
        c = 7
    else:
        d = [abs(g - a) for g in grid]
        m = min(d)
        best = [i for i, di in enumerate(d) if di == m]
        c = [i for i in best if i % 2 == 0][0] if len(best) > 1 else best[0]
    return c | (8 if np.signbit(x) else 0)


def test_e2m1_encode_brute_force():
    pts = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 100], np.float32)
    sweep = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0)),
                            np.linspace(0, 8, 4001, dtype=np.float32)])
    sweep = np.concatenate([sweep, -sweep, np.float32([-0.0])])
    got = F.e2m1_encode(sweep)
    want = np.array([_e2m1_brute(x) for x in sweep], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e2m1_decode_table():
    v = F.e2m1_decode(np.arange(16))
    assert list(v[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(v[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


# ---------------------------------------------------------------- int4 / packing
def test_int4_nibbles_roundtrip():
    q = np.arange(-7, 8)
    n = F.int4_to_nibble(q)
    assert list(n[:7]) == [15, 14, 13, 12, 11, 10, 9]
    assert list(n[7:]) == [0, 1, 2, 3, 4, 5, 6, 7]
    assert np.array_equal(F.nibble_to_int4(n), q)
    assert F.nibble_to_int4(np.array([8]))[0] == 0
    with pytest.raises(ValueError):
        F.int4_to_nibble(np.array([-8]))


def test_pack_layout_low_nibble_even():
    codes = np.array([[1, 2, 3, 4]], np.uint8)
    assert list(F.pack_nibbles(codes)[0]) == [0x21, 0x43]


@settings(max_examples=50, deadline=None)
@given(st.integers(1, 5), st.integers(1, 20), st.integers(0, 2 ** 31 - 1))
def test_pack_unpack_roundtrip(r, k2, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 16, size=(r, 2 * k2)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)
