"""Pins for oracle/quant.py: closed-form scales, exact recovery of data already
on the 4-bit grid, power-of-two invariance, zero groups, nearest-integer
optimality of the codes, and the AWQ zero-point tie rule."""

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import formats as F, quant as Q

F32 = np.float32


def test_int4_scale_closed_form():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((5, 256)) * 3).astype(F32)
    nib, s, q = Q.quantize_int4(x, 64)
    amax = np.abs(x.reshape(5, 4, 64)).max(axis=2)
    # s is bf16(amax/7): within half a bf16 ulp of the real quotient
    rel = np.abs(s.astype(np.float64) - amax / 7.0) / (amax / 7.0)
    assert rel.max() <= 2.0 ** -8 + 1e-7
    assert np.array_equal(F.bf16_round(s), s)
    assert np.abs(q).max() <= 7 and np.abs(q).max() == 7


def test_int4_codes_are_nearest_integers():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((16, 512)) * rng.uniform(0.01, 100, (16, 1))).astype(F32)
    _, s, q = Q.quantize_int4(x, 64)
    ratio = x.reshape(16, 8, 64).astype(np.float64) / s[..., None].astype(np.float64)
    # nearest integer to the exact quotient, up to the fp32 rounding of x*(1/s)
    d = np.abs(q.reshape(16, 8, 64) - ratio)
    assert d.max() <= 0.5 + 1e-6


def test_int4_exact_recovery():
    rng = np.random.default_rng(2)
    q = rng.integers(-7, 8, size=(8, 256))
    q[:, ::64] = 7 * rng.choice([-1, 1], size=(8, 4))  # every group holds +-7
    e = rng.integers(-20, 20, size=(8, 4))
    x = (q.reshape(8, 4, 64) * np.ldexp(1.0, e)[..., None]).reshape(8, 256).astype(F32)
    nib, s, q2 = Q.quantize_int4(x, 64)
    assert np.array_equal(q2, q)
    assert np.array_equal(s, np.ldexp(1.0, e).astype(F32))
    assert np.array_equal(F.nibble_to_int4(nib), q)


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.integers(-30, 30))
def test_int4_power_of_two_invariance(seed, j):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 128)) * 2).astype(F32)
    n1, s1, _ = Q.quantize_int4(x, 64)
    n2, s2, _ = Q.quantize_int4((x * F32(2.0 ** j)).astype(F32), 64)
    assert np.array_equal(n1, n2)
    assert np.array_equal(s2, (s1 * F32(2.0 ** j)).astype(F32))


def test_int4_zero_groups():
    x = np.zeros((2, 128), F32)
    x[1, 64:] = 1e-35  # amax below 2^-100
    x[0, 64] = -0.0
    nib, s, q = Q.quantize_int4(x, 64)
    assert not nib.any() and not s.any() and not q.any()


def test_int4_sign_of_zero_codes():
    x = np.zeros((1, 64), F32)
    x[0, 0] = 7.0
    x[0, 1] = -0.1  # rounds to magnitude 0, keeps its sign bit
    nib, _, q = Q.quantize_int4(x, 64)
    assert nib[0, 1] == 8 and q[0, 1] == 0 and nib[0, 2] == 0


# ---------------------------------------------------------------- nvfp4
def test_nvfp4_act_exact_recovery():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(4, 64)).astype(np.uint8)
    codes[:, ::16] = 7 | (rng.integers(0, 2, size=(4, 4)) << 3)  # a +-6 in every group
    s8 = rng.integers(0x08, 0x77, size=(4, 4)).astype(np.uint8)  # E4M3 scales (normal)
    S = F.e4m3_decode(s8).astype(np.float64)
    x = (F.e2m1_decode(codes).reshape(4, 4, 16) * S[..., None]).reshape(4, 64).astype(F32)
    c2, s82 = Q.quantize_nvfp4_act(x, 16)
    assert np.array_equal(s82, s8)
    # +-0 codes may differ only in the sign of zero (value 0 either way)
    v1 = F.e2m1_decode(c2)
    assert np.array_equal(v1, F.e2m1_decode(codes))


def test_nvfp4_act_scale_closed_form():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((6, 128)) * 5).astype(F32)
    _, s8 = Q.quantize_nvfp4_act(x, 16)
    amax = np.abs(x.reshape(6, 8, 16)).max(axis=2).astype(F32)
    assert np.array_equal(s8, F.e4m3_encode((amax / F32(6)).astype(F32)))


def test_nvfp4_weight_tensor_scale_and_recovery():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(4, 64)).astype(np.uint8)
    codes[:, ::16] = 7
    s8 = rng.integers(0x08, 0x77, size=(4, 4)).astype(np.uint8)
    s8[0, 0] = 0x7E  # 448: this block's amax is 6 * 448 = 2688, so t_w = 1
    S = F.e4m3_decode(s8).astype(np.float64)
    w = (F.e2m1_decode(codes).reshape(4, 4, 16) * S[..., None]).reshape(4, 64).astype(F32)
    c2, s82, t = Q.quantize_nvfp4_weight(w, 16)
    assert t == 1.0
    assert np.array_equal(s82, s8)
    assert np.array_equal(F.e2m1_decode(c2), F.e2m1_decode(codes))


def test_nvfp4_weight_tensor_scale_closed_form():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(F32)
    _, _, t = Q.quantize_nvfp4_weight(w, 16)
    assert t == float(F32(np.abs(w).max() / F32(2688)))


def test_nvfp4_zero_and_tiny():
    codes, s8 = Q.quantize_nvfp4_act(np.zeros((1, 32), F32), 16)
    assert not codes.any() and not s8.any()
    x = np.full((1, 16), 1e-4, F32)  # amax/6 < 2^-10 rounds to a zero E4M3 scale
    codes, s8 = Q.quantize_nvfp4_act(x, 16)
    assert not codes.any() and not s8.any()
    c, s, t = Q.quantize_nvfp4_weight(np.zeros((2, 16), F32), 16)
    assert t == 1.0 and not c.any() and not s.any()


# ---------------------------------------------------------------- AWQ
def test_awq_exact_recovery():
    rng = np.random.default_rng(7)
    N, K = 6, 192
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::64] = 0
    q[:, 1::64] = 15
    z = rng.integers(0, 16, size=(N, K // 64))
    e = rng.integers(-12, 0, size=(N, K // 64))
    s = np.ldexp(1.0, e)
    w = ((q.reshape(N, 3, 64) - z[..., None]) * s[..., None]).reshape(N, K).astype(F32)
    q2, s2, z2 = Q.quantize_awq(w, 64)
    assert np.array_equal(s2, s.astype(F32))
    assert np.array_equal(z2, z.astype(F32))
    assert np.array_equal(q2, q)


def test_awq_range_includes_zero():
    w = np.full((1, 64), 3.0, F32)
    w[0, 0] = 1.5
    q, s, z = Q.quantize_awq(w, 64)
    assert z[0, 0] == 0  # min clamps to 0
    assert s[0, 0] == F.bf16_round(np.float32([3.0 / 15]))[0]


def test_awq_zero_point_tie_rule():
    # q = rne(w/s) + z, not rne(w/s + z): with z odd, x/s = 0.5 rounds to 0 then shifts
    s = 1.0
    w = np.zeros((1, 64), F32)
    w[0, 0] = -3.0     # wmin -> z = 3 (odd)
    w[0, 1] = 12.0     # wmax -> range 15, s = 1
    w[0, 2] = 0.5      # exact tie
    q, s2, z = Q.quantize_awq(w, 64)
    assert s2[0, 0] == s and z[0, 0] == 3
    assert q[0, 2] == 3  # rne(0.5) = 0, + 3
    # (rne(0.5 + 3) would give 4)


def test_awq_codes_nearest():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((32, 256)) * 0.02).astype(F32)
    q, s, z = Q.quantize_awq(w, 64)
    deq = (q.reshape(32, 4, 64) - z[..., None]) * s[..., None].astype(np.float64)
    err = np.abs(deq - w.reshape(32, 4, 64))
    qq = q.reshape(32, 4, 64)
    inner = (qq > 0) & (qq < 15)  # not clamped: nearest grid point
    sb = np.broadcast_to(s[..., None].astype(np.float64), err.shape)
    assert np.all(err[inner] <= 0.5 * sb[inner] * (1 + 2e-6))
    # clamped ends: s may sit up to 2^-8 below range/15 and z is rounded, so the
    # end points can be off by at most one step plus that shortfall
    assert np.all(err <= sb * (1 + 15 * 2.0 ** -8) + 1e-30)
