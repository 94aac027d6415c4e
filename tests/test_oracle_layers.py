"""Pins for oracle/layers.py: brute-force integer GEMMs on 8x16x16 inputs,
Eckart-Young-Mirsky for the low-rank split, exact zero-residual recovery,
smoothing and reconstruction identities, zero/permutation identities, the AWQ
reference against a Python loop, and the method's premise (SVDQ beats plain
W4A4 on outlier-heavy inputs)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synthetic as S
from oracle import formats as F, layers as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ones_smooth(K):
    return F.bf16_bits(np.ones(K, np.float32))


# ------------------------------------------------------------ brute-force GEMM
def _decode_nibble_int4(b):
    mag = b & 7
    return -mag if b & 8 else mag


def _decode_nibble_e2m1_doubled(b):
    mag = [0, 1, 2, 3, 4, 6, 8, 12][b & 7]
    return -mag if b & 8 else mag


def _brute_partials(packed_a, packed_w, G, dec):
    """Python-int triple loop over bytes of the packed operands."""
    M, K2 = packed_a.shape
    N = packed_w.shape[0]
    K = 2 * K2
    P = [[[0] * (K // G) for _ in range(N)] for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for k in range(K):
                ba = int(packed_a[m, k // 2])
                bw = int(packed_w[n, k // 2])
                na = ba & 15 if k % 2 == 0 else ba >> 4
                nw = bw & 15 if k % 2 == 0 else bw >> 4
                P[m][n][k // G] += dec(na) * dec(nw)
    return np.array(P, dtype=np.int64)


@pytest.mark.parametrize("precision,K", [("nvfp4", 16), ("int4", 64), ("int4", 128), ("nvfp4", 48)])
def test_partials_and_output_brute_force(precision, K):
    M, N = 8, 16
    rng = np.random.default_rng(K)
    x = S.to_bf16_bits(rng.standard_normal((M, K)) * 2)
    w = rng.standard_normal((N, K)) * 0.1
    b = S.to_bf16_bits(rng.standard_normal(N) * 0.01)
    lay = L.prepare_svdq_layer(w, _ones_smooth(K), 0, precision, b)
    act = L.svdq_quantize_act(x, lay["smooth"], lay["lora_down"], precision)
    G = L.GROUP[precision]
    dec = _decode_nibble_int4 if precision == "int4" else _decode_nibble_e2m1_doubled
    Pb = _brute_partials(act["packed"], lay["packed_w"], G, dec)
    assert np.array_equal(L.svdq_partials_ref(act["codes"], lay["w_codes"], precision), Pb)
    # output in exact rational arithmetic from the brute-force partials
    sa = act["scales"]
    sw = lay["wscales"]
    sdec = (lambda v: Fraction(float(F.bf16_to_f32(np.uint16(v))))) if precision == "int4" else \
        (lambda v: Fraction(float(F.e4m3_decode(np.uint8(v)))))
    c = Fraction(1) if precision == "int4" else Fraction(lay["wtscale"]) / 4
    y = L.svdq_linear_ref(x, lay)
    for m in range(M):
        for n in range(N):
            acc = Fraction(float(F.bf16_to_f32(b[n])))
            for g in range(K // G):
                acc += int(Pb[m, n, g]) * sdec(sa[m, g]) * sdec(sw[n, g]) * c
            assert abs(float(acc) - y[m, n]) <= 1e-12 * (1 + abs(float(acc)))


def test_awq_reference_brute_force():
    rng = np.random.default_rng(3)
    N, K, M = 8, 128, 3
    w = rng.standard_normal((N, K)) * 0.05
    lay = L.prepare_awq_layer(w, S.to_bf16_bits(rng.standard_normal(N) * 0.01))
    x = S.to_bf16_bits(rng.standard_normal((M, K)))
    y = L.awq_linear_ref(x, lay)
    for m in range(M):
        for n in range(N):
            acc = Fraction(float(F.bf16_to_f32(lay["bias"][n])))
            for k in range(K):
                byte = int(lay["packed_w"][n, k // 2])
                q = byte & 15 if k % 2 == 0 else byte >> 4
                s = Fraction(float(F.bf16_to_f32(lay["wscales"][n, k // 64])))
                z = Fraction(float(F.bf16_to_f32(lay["wzeros"][n, k // 64])))
                acc += Fraction(float(F.bf16_to_f32(x[m, k]))) * (q - z) * s
            assert abs(float(acc) - y[m, n]) <= 1e-12 * (1 + abs(float(acc)))


# ------------------------------------------------------------ low-rank split
def _known_spectrum(N, K, sig, rng):
    u, _ = np.linalg.qr(rng.standard_normal((N, len(sig))))
    v, _ = np.linalg.qr(rng.standard_normal((K, len(sig))))
    return (u * sig) @ v.T


def test_svd_split_eckart_young():
    rng = np.random.default_rng(4)
    N, K, r = 96, 128, 8
    sig = np.sort(rng.uniform(0.1, 3.0, 40))[::-1]
    w = _known_spectrum(N, K, sig, rng)
    lay = L.prepare_svdq_layer(w, _ones_smooth(K), r, "int4")
    assert np.allclose(lay["sigma"][:40], sig, rtol=1e-10, atol=1e-12)
    assert np.all(lay["sigma"][40:] < 1e-10)
    tail = np.sqrt(np.sum(sig[r:] ** 2))
    head = np.sqrt(np.sum(sig[:r] ** 2))
    fro = np.linalg.norm(lay["resid"])
    # the factors are rounded to bf16, which perturbs the split by <= ~2^-8 of the head
    assert abs(fro - tail) <= 2.0 ** -6 * head
    assert fro >= tail * (1 - 1e-9)  # no rank-r matrix beats the tail
    up = F.bf16_to_f32(lay["lora_up"]).astype(np.float64)
    gram = up.T @ up
    assert np.allclose(gram, np.eye(r), atol=2.0 ** -6)


def test_zero_residual_exact():
    # W with exactly bf16-representable rank-r factors (scaled permutations):
    # the split is exact, the residual is 0, all weight codes are 0, and the
    # output is exactly X_hat lora_down^T lora_up^T + bias.
    rng = np.random.default_rng(5)
    N, K, r = 64, 128, 4
    sig = np.array([8.0, 4.0, 2.0, 1.0])
    rows = rng.choice(N, r, replace=False)
    cols = rng.choice(K, r, replace=False)
    w = np.zeros((N, K))
    w[rows, cols] = sig
    x = S.to_bf16_bits(rng.standard_normal((5, K)))
    for p in ("int4", "nvfp4"):
        lay = L.prepare_svdq_layer(w, _ones_smooth(K), r, p)
        assert np.abs(lay["resid"]).max() < 1e-12
        assert not lay["packed_w"].any()
        y = L.svdq_linear_ref(x, lay)
        xf = F.bf16_to_f32(x).astype(np.float64)
        assert np.allclose(y, xf @ w.T, rtol=0, atol=1e-12)


def test_reconstruction_identity():
    rng = np.random.default_rng(6)
    N, K = 64, 128
    w = rng.standard_normal((N, K)) * 0.02
    sm = S.to_bf16_bits(rng.uniform(0.5, 3, K))
    lay = L.prepare_svdq_layer(w, sm, 16, "int4")
    up = F.bf16_to_f32(lay["lora_up"]).astype(np.float64)
    dn = F.bf16_to_f32(lay["lora_down"]).astype(np.float64)
    smooth = F.bf16_to_f32(sm).astype(np.float64)
    assert np.allclose(up @ dn + lay["resid"], w * smooth[None, :], rtol=0, atol=1e-15)


def test_smoothing_identity():
    rng = np.random.default_rng(7)
    M, N, K = 16, 32, 128
    x = S.to_bf16_bits(rng.standard_normal((M, K)) * 3)
    w = rng.standard_normal((N, K)) * 0.02
    sm = L.smooth_factors(x, w)
    xf = F.bf16_to_f32(x).astype(np.float64)
    lam = F.bf16_to_f32(sm).astype(np.float64)
    # closed form of the calibration, up to the bf16 rounding of lambda
    ref = np.sqrt(np.abs(xf).max(0) / np.abs(w).max(0))
    assert np.all(np.abs(lam - ref) <= 2.0 ** -8 * ref)
    xhat = L.smoothed_activations(x, sm).astype(np.float64)
    lay = L.prepare_svdq_layer(w, sm, 0, "int4")
    # (X / lambda)(W lambda)^T = X W^T, up to the fp32 rounding of X_hat
    assert np.allclose(xhat @ lay["w_hat"].T, xf @ w.T, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------ identities
@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_zero_weight_and_zero_input(precision):
    rng = np.random.default_rng(8)
    M, N, K = 6, 32, 128
    x = S.to_bf16_bits(rng.standard_normal((M, K)))
    b = S.to_bf16_bits(rng.standard_normal(N) * 0.01)
    lay = L.prepare_svdq_layer(np.zeros((N, K)), _ones_smooth(K), 0, precision)
    assert not L.svdq_linear_ref(x, lay).any()
    w = rng.standard_normal((N, K)) * 0.02
    lay = L.prepare_svdq_layer(w, _ones_smooth(K), 16, precision, b)
    y = L.svdq_linear_ref(np.zeros((M, K), np.uint16), lay)
    assert np.array_equal(y, np.broadcast_to(F.bf16_to_f32(b).astype(np.float64), (M, N)))


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_row_permutation_equivariance(precision):
    rng = np.random.default_rng(9)
    M, N, K = 12, 32, 128
    x = S.to_bf16_bits(rng.standard_normal((M, K)) * 2)
    w = rng.standard_normal((N, K)) * 0.02
    lay = L.prepare_svdq_layer(w, _ones_smooth(K), 16, precision)
    perm = rng.permutation(M)
    a1 = L.svdq_quantize_act(x, lay["smooth"], lay["lora_down"], precision)
    a2 = L.svdq_quantize_act(x[perm], lay["smooth"], lay["lora_down"], precision)
    assert np.array_equal(a1["codes"][perm], a2["codes"])
    assert np.array_equal(a1["scales"][perm], a2["scales"])
    assert np.array_equal(L.svdq_linear_ref(x, lay)[perm], L.svdq_linear_ref(x[perm], lay))


def test_method_premise_svdq_beats_plain_w4a4():
    # outlier channels + a low-rank spike: smoothing + rank-32 branch must reduce
    # the error of 4-bit quantization (the news article's account of SVDQuant)
    c = S.config1(seed=3, M=256, K=512, N=512)
    xf = F.bf16_to_f32(c["x"]).astype(np.float64)
    exact = xf @ c["w"].T
    plain = L.prepare_svdq_layer(c["w"], _ones_smooth(512), 0, "int4")
    sm = L.smooth_factors(c["x"], c["w"])
    svdq = L.prepare_svdq_layer(c["w"], sm, 32, "int4")
    e_plain = np.linalg.norm(L.svdq_linear_ref(c["x"], plain) - exact)
    e_svdq = np.linalg.norm(L.svdq_linear_ref(c["x"], svdq) - exact)
    assert e_svdq < 0.6 * e_plain


# ------------------------------------------------------------ the pages' table
def test_group_sizes_match_the_pages_table():
    tab = json.load(open(os.path.join(GOLDEN, "quantization_types.json")))
    svdq = {r["precision"]: r["group_size"] for r in tab["rows"] if r["method"] == "svdq_w4a4"}
    assert svdq == L.GROUP
    awq = [r for r in tab["rows"] if r["method"] == "awq_w4a16"]
    assert awq == [{"method": "awq_w4a16", "precision": "int4", "group_size": 64}]
    ex = json.load(open(os.path.join(GOLDEN, "config_example.json")))
    assert ex["svdq"]["group_size"] == L.GROUP[ex["svdq"]["precision"]]
    assert ex["compute_dtype"] == "bfloat16"


# ------------------------------------------------------------------ GELU (MLP fusion)
def test_gelu_identities():
    # gelu(y) - gelu(-y) = y (the erf term is odd), gelu(0) = 0, and
    # gelu(y) -> y for large y, gelu(y) -> 0 for large negative y
    y = np.linspace(-8, 8, 4001)
    assert np.allclose(L.gelu_f64(y) - L.gelu_f64(-y), y, rtol=0, atol=1e-14)
    assert L.gelu_f64(np.array([0.0]))[0] == 0.0
    assert np.allclose(L.gelu_f64(np.array([30.0, -30.0])), [30.0, 0.0], rtol=0, atol=1e-12)
    # closed form at y = sqrt(2): sqrt(2)/2 (1 + erf(1)), erf(1) = 0.8427007929497149
    assert abs(L.gelu_f64(np.array([np.sqrt(2.0)]))[0] - np.sqrt(2.0) / 2 * (1 + 0.8427007929497149)) < 1e-15


def test_gelu_matches_high_precision():
    # the definition y/2 (1 + erf(y / sqrt 2)) evaluated with mpmath at 90
    # digits (enough to survive the cancellation of 1 + erf down to y = -14),
    # on every finite bf16 value with |y| < 14; beyond, the negative tail lies
    # below the bf16 range and the positive one equals y
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 90
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(bits)
    bits = bits[np.isfinite(v) & (np.abs(v) < 14)]
    y = F.bf16_to_f32(bits).astype(np.float64)
    exact = np.array([float(mp.mpf(t) / 2 * (1 + mp.erf(mp.mpf(t) / mp.sqrt(2)))) for t in y])
    got = L.gelu_f64(y)
    scale = np.maximum(np.abs(exact), 1e-300)
    assert np.max(np.abs(got - exact) / scale) < 1e-13  # scipy erfc: a few 1e-14 in the far tail
    # bf16: one rounding of the correctly rounded value, equal bits (a tie
    # between the two fp64 values and a bf16 boundary aside; mpmath's zero is
    # unsigned, gelu(-0) = -0)
    assert (L.gelu_bf16(bits) != F.bf16_bits_f64(exact)).sum() <= 1
    tail = np.array([-14.0, -20.0, -63.5])
    assert np.all(np.abs(L.gelu_f64(tail)) < 2.0 ** -130)
    assert np.array_equal(L.gelu_f64(np.array([14.0, 20.0, 63.5])), [14.0, 20.0, 63.5])


def test_gelu_matches_torch():
    # torch's exact-erf GELU in float64 (a library routine), where its 1 + erf
    # form keeps full accuracy (y >= -4)
    torch = pytest.importorskip("torch")
    y = np.random.default_rng(0).uniform(-4, 8, 20000)
    ref = torch.nn.functional.gelu(torch.from_numpy(y), approximate="none").numpy()
    assert np.allclose(L.gelu_f64(y), ref, rtol=1e-11, atol=1e-300)


# ------------------------------------------------------------------ QKV + RMSNorm + RoPE
def test_rope_matches_complex_rotation():
    # interleaved pairs as complex numbers a + ib times e^{i theta}
    rng = np.random.default_rng(3)
    n = rng.standard_normal((5, 4, 16))
    th = rng.uniform(-40, 40, (5, 1, 8))
    got = L.rope_f64(n, np.cos(th), np.sin(th))
    z = (n[..., 0::2] + 1j * n[..., 1::2]) * np.exp(1j * th)
    assert np.allclose(got[..., 0::2], z.real, rtol=0, atol=1e-12)
    assert np.allclose(got[..., 1::2], z.imag, rtol=0, atol=1e-12)


def test_rope_identities():
    rng = np.random.default_rng(4)
    n = rng.standard_normal((3, 8))
    assert np.array_equal(L.rope_f64(n, np.ones((3, 4)), np.zeros((3, 4))), n)
    # quarter turn: (a, b) -> (-b, a)
    q = L.rope_f64(n, np.zeros((3, 4)), np.ones((3, 4)))
    assert np.array_equal(q[:, 0::2], -n[:, 1::2]) and np.array_equal(q[:, 1::2], n[:, 0::2])
    # pair norms are kept; rotations compose
    a, b = rng.uniform(-3, 3, (3, 4)), rng.uniform(-3, 3, (3, 4))
    r1 = L.rope_f64(L.rope_f64(n, np.cos(a), np.sin(a)), np.cos(b), np.sin(b))
    r2 = L.rope_f64(n, np.cos(a + b), np.sin(a + b))
    assert np.allclose(r1, r2, atol=1e-12)
    assert np.allclose(r1[:, 0::2] ** 2 + r1[:, 1::2] ** 2, n[:, 0::2] ** 2 + n[:, 1::2] ** 2, atol=1e-12)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(5)
    one = np.full(64, 0x3F80, np.uint16)
    h = S.to_bf16_bits(rng.standard_normal((6, 64)) * 3.0)
    n = F.bf16_to_f32(L.rmsnorm_bf16(h, one, 0.0)).astype(np.float64)
    # unit weight: every row has mean square 1, up to the bf16 rounding
    assert np.allclose(np.mean(n * n, axis=1), 1.0, atol=2 * 2.0 ** -8)
    # scale invariance (eps = 0): powers of two change nothing, bit for bit
    h4 = F.bf16_bits_f64(F.bf16_to_f32(h).astype(np.float64) * 4.0)
    assert np.array_equal(L.rmsnorm_bf16(h4, one, 0.0), L.rmsnorm_bf16(h, one, 0.0))
    # a constant row c gives c / sqrt(c^2 + eps) * w
    w = S.to_bf16_bits(rng.uniform(0.5, 1.5, 64))
    c = F.bf16_bits_f64(np.full((1, 64), -0.375))
    got = F.bf16_to_f32(L.rmsnorm_bf16(c, w, 1e-6)).astype(np.float64)
    want = F.bf16_to_f32(F.bf16_bits_f64(-0.375 / np.sqrt(0.375 ** 2 + 1e-6) * F.bf16_to_f32(w))).astype(np.float64)
    assert np.array_equal(got[0], want)


def test_qkv_norm_rope_brute_force():
    # per token, head and pair with scalar math on a tiny layer
    import math
    rng = np.random.default_rng(6)
    M, K, H, D = 3, 128, 2, 8
    x = S.activations(M, K, 1, rng)
    lay = L.prepare_svdq_layer(S.weight(3 * H * D, K, 0.05, rng), np.full(K, 0x3F80, np.uint16), 16, "nvfp4",
                               S.bias(3 * H * D, rng))
    qw, kw = S.norm_weight(D, rng), S.norm_weight(D, rng)
    cos, sin = S.rope_tables(M, D, offset=7)
    eps = 1e-6
    got = L.qkv_norm_rope_ref(x, lay, H, qw, kw, eps, cos, sin)
    h64 = L.svdq_linear_ref(x, lay)
    hb = F.bf16_to_f32(F.bf16_bits_f64(h64)).astype(np.float64)
    f = lambda bits: float(F.bf16_to_f32(np.array([bits], np.uint16))[0])
    rnd = lambda v: f(F.bf16_bits_f64(np.array([v]))[0])
    for m in range(M):
        for part, wb in ((0, qw), (1, kw)):
            for hd in range(H):
                c0 = (part * H + hd) * D
                vals = [hb[m, c0 + d] for d in range(D)]
                ms = sum(v * v for v in vals) / D
                nv = [rnd(vals[d] / math.sqrt(ms + eps) * f(wb[d])) for d in range(D)]
                for i in range(D // 2):
                    a, b = nv[2 * i], nv[2 * i + 1]
                    cs, sn = float(cos[m, i]), float(sin[m, i])
                    assert math.isclose(got[m, c0 + 2 * i], a * cs - b * sn, rel_tol=0, abs_tol=1e-12)
                    assert math.isclose(got[m, c0 + 2 * i + 1], a * sn + b * cs, rel_tol=0, abs_tol=1e-12)
        assert np.array_equal(got[m, 2 * H * D:], h64[m, 2 * H * D:])


def test_low_rank_residual_against_exact_arithmetic():
    # R = W_hat - up down with the rank terms added in order: against
    # Fraction arithmetic, the error is at most r + 1 roundings of the
    # largest partial sum; with factors on a common power-of-two grid every
    # partial sum is exact and so is R
    from fractions import Fraction
    rng = np.random.default_rng(12)
    N, K, r = 6, 8, 5
    w = F.bf16_round(rng.standard_normal((N, K)).astype(np.float32)).astype(np.float64)
    sm = F.bf16_bits(rng.uniform(0.5, 2, K).astype(np.float32))
    up = F.bf16_bits(rng.standard_normal((N, r)).astype(np.float32))
    dn = F.bf16_bits(rng.standard_normal((r, K)).astype(np.float32))
    w_hat, R = L.low_rank_residual(w, sm, dn, up)
    upf, dnf, smf = (F.bf16_to_f32(a).astype(np.float64) for a in (up, dn, sm))
    for n in range(N):
        for k in range(K):
            wh = Fraction(w[n, k]) * Fraction(smf[k])
            assert Fraction(w_hat[n, k]) == wh            # the product is exact
            exact = wh - sum(Fraction(upf[n, j]) * Fraction(dnf[j, k]) for j in range(r))
            big = max([abs(wh)] + [abs(Fraction(upf[n, j]) * Fraction(dnf[j, k])) for j in range(r)])
            assert abs(Fraction(R[n, k]) - exact) <= (r + 1) * r * big * Fraction(2) ** -53
    # small-integer factors times 2^-4: every partial sum is exact
    up2 = F.bf16_bits((rng.integers(-8, 8, (N, r)) / 16).astype(np.float32))
    dn2 = F.bf16_bits((rng.integers(-8, 8, (r, K)) / 16).astype(np.float32))
    ones = F.bf16_bits(np.ones(K, np.float32))
    _, R2 = L.low_rank_residual(w, ones, dn2, up2)
    u2, d2 = F.bf16_to_f32(up2).astype(np.float64), F.bf16_to_f32(dn2).astype(np.float64)
    for n in range(N):
        for k in range(K):
            exact = Fraction(w[n, k]) - sum(Fraction(u2[n, j]) * Fraction(d2[j, k]) for j in range(r))
            assert Fraction(R2[n, k]) == exact


def test_prepare_from_factors_reproduces_prepare():
    # the split of prepare_svdq_layer is the composition of the SVD and
    # prepare_svdq_layer_from_factors
    rng = np.random.default_rng(13)
    w = S.weight(96, 256, 0.02, rng, spike_rank=2)
    sm = F.bf16_bits(rng.uniform(0.5, 2, 256).astype(np.float32))
    for p in ("int4", "nvfp4"):
        a = L.prepare_svdq_layer(w, sm, 16, p)
        b = L.prepare_svdq_layer_from_factors(w, sm, a["lora_down"], a["lora_up"], p)
        for key in ("packed_w", "wscales", "resid"):
            assert np.array_equal(a[key], b[key]), key
        assert a["wtscale"] == b["wtscale"]


# ------------------------------------------- nvfp4 activation range (tensor scale 1)
def test_nvfp4_activation_range_low_magnitude_rows():
    # With tensor scale 1 an activation group's E4M3 scale is E4M3(amax / 6):
    # it rounds to zero when amax / 6 <= 2^-10 (half the smallest subnormal
    # 2^-9, ties to even), i.e. amax <= 6 * 2^-10.  Such a group gets scale 0
    # and all-zero codes, so a row whose groups all lie below that bound keeps
    # only its 16-bit low-rank branch and the bias.  Above the bound the row's
    # relative error stays of the order it has at unit magnitude.
    rng = np.random.default_rng(17)
    K, N, r = 256, 64, 16
    w = S.weight(N, K, 0.05, rng, spike_rank=2)
    lay = L.prepare_svdq_layer(w, _ones_smooth(K), r, "nvfp4", bias_bits=S.bias(N, rng))
    # unit row: every 16-value group has amax exactly 1
    u = rng.uniform(-1.0, 1.0, (4, K)).astype(np.float32)
    u[:, ::16] = np.where(rng.random((4, K // 16)) < 0.5, -1.0, 1.0)
    up = F.bf16_to_f32(lay["lora_up"]).astype(np.float64)
    bias = F.bf16_to_f32(lay["bias"]).astype(np.float64)
    err = {}
    for e in (0, 4, 7, 8, 12):
        x_bits = F.bf16_bits(u * np.float32(2.0 ** -e))  # exact: power-of-two scaling of bf16 values
        xf = F.bf16_to_f32(x_bits).astype(np.float64)
        act = L.svdq_quantize_act(x_bits, lay["smooth"], lay["lora_down"], "nvfp4")
        y = L.svdq_linear_ref(x_bits, lay, act)
        exact = xf @ w.T
        err[e] = np.linalg.norm(y - bias - exact) / np.linalg.norm(exact)
        if 2.0 ** -e <= 6 * 2.0 ** -10:
            # below the range: zero scales and codes, low rank + bias only
            assert not act["scales"].any() and not act["codes"].any()
            np.testing.assert_array_equal(y, act["lora_act"] @ up.T + bias[None, :])
        else:
            assert act["scales"].all()
    print({k: f"{v:.3e}" for k, v in err.items()})
    # inside the range (amax 2^-7 uses the subnormal scale 2^-9) the error is
    # of the unit row's order; below it the residual branch is lost
    assert err[4] <= 1.5 * err[0] and err[7] <= 3.0 * err[0]
    assert err[8] > err[0] and err[12] > err[0]
