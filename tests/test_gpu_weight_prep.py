"""GPU weight preparation against the oracle's packer, bit for bit.

svdq_w4a4_smooth_factors and svdq_w4a4_pack_weight must give exactly the
oracle's smoothing factors, codes, scales and tensor scale on the same
inputs (fp32 weights and residuals); the GPU-prepared layer (with torch's
randomized SVD for the low-rank split) must be as accurate as the
oracle-prepared one.
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F, layers as L, quant as Q

bq = pytest.importorskip("bit_quantized_linear_quantize_amd")

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_smooth_factors_bit_exact():
    rng = np.random.default_rng(41)
    M, N, K = 300, 768, 1024
    x = S.activations(M, K, 10, rng)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xf = F.bf16_to_f32(x).copy()
    xf[:, 1] = 0.0                         # zero activation column: factor 1
    w[:, 0] = 0.0                          # zero weight column: factor 1
    w[:, 2] = 1e-30                        # huge ratio
    w[5, 3] = 3e38                         # tiny ratio
    xf[:, 4] = 2.0 ** -133                 # bf16 subnormal activations
    w[:, 4] = 3e38                         # -> a bf16-subnormal factor
    xf[7, 5] = -2.0 ** 100                 # negative maxima count by magnitude
    x = F.bf16_bits_f64(xf.astype(np.float64))
    got = host_bits(bq.smooth_factors(dev_bf16(x), dev(w)))
    want = L.smooth_factors(x, w.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(int(k), int(got[k]), int(want[k])) for k in bad[:8]]
    assert got[0] == 0x3F80 and got[1] == 0x3F80


def _residual(N, K, rng, precision):
    r = (rng.standard_normal((N, K)) * 0.01).astype(np.float32)
    G = 64 if precision == "int4" else 16
    r[0, :G] = 0.0                                   # zero group
    r[1, :G] = 1e-31                                 # below 2^-100: a zero group
    r[2, :G] = -0.0                                  # negative zeros
    r[3, :G] = 2.0 ** -140                           # fp32 subnormals
    if precision == "int4":
        # ties of rne(x / s): s = 2^-7 (amax = 7 s), values (q + 1/2) s
        q = rng.integers(-6, 6, G)
        r[4, :G] = (q + 0.5) * 2.0 ** -7
        r[4, 0] = 7 * 2.0 ** -7
    else:
        # E2M1 midpoints (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) times S = 2^-6:
        # the largest group below makes t = 168 / 2688 = 2^-4, and this
        # group's amax 6 S gives s8 = E4M3(0.25) exactly
        r[4, :16] = np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 0]) * 2.0 ** -6
    # one large group, amax 168 (the tensor maximum)
    r[5, G:2 * G] = np.clip(r[5, G:2 * G] * 1e4, -160, 160)
    r[5, G] = -168.0
    return r


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("N,K", [(384, 1024), (9216, 3072)])
def test_pack_weight_bit_exact(precision, N, K):
    rng = np.random.default_rng(N + K)
    r = _residual(N, K, rng, precision)
    packed, wscales, wt = bq.pack_weight(dev(r), precision)
    torch.cuda.synchronize()
    if precision == "int4":
        nib, s, _ = Q.quantize_int4(r, 64)
        want_sc, t = F.bf16_bits(s), 1.0
        got_sc = host_bits(wscales)
    else:
        nib, want_sc, t = Q.quantize_nvfp4_weight(r, 16)
        got_sc = wscales.cpu().numpy()
    want_pk = F.pack_nibbles(nib)
    got_pk = packed.cpu().numpy()
    bad = np.argwhere(got_pk != want_pk)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first {bad[:4].tolist()}"
    assert np.array_equal(got_sc, want_sc)
    assert np.float32(wt.cpu().numpy()[0]) == np.float32(t)


def test_pack_weight_zero_tensor():
    r = np.zeros((64, 256), np.float32)
    packed, wscales, wt = bq.pack_weight(dev(r), "nvfp4")
    assert not packed.any() and not wscales.any() and float(wt.cpu()[0]) == 1.0


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_prepare_layer_on_gpu(precision):
    # the GPU-prepared layer is as accurate as the oracle-prepared one
    rng = np.random.default_rng(7)
    M, K, N = 256, 1024, 768
    x = S.activations(M, K, 10, rng)
    w = S.weight(N, K, 0.02, rng, spike_rank=4).astype(np.float32)
    b = S.bias(N, rng)
    exact = F.bf16_to_f32(x).astype(np.float64) @ w.astype(np.float64).T + F.bf16_to_f32(b).astype(np.float64)
    xd = dev_bf16(x)
    layer = bq.prepare_layer(dev(w), xd, 32, precision, bias=dev_bf16(b))
    assert np.array_equal(host_bits(layer.smooth), L.smooth_factors(x, w.astype(np.float64)))
    y_gpu = F.bf16_to_f32(host_bits(layer(xd))).astype(np.float64)
    lay = L.prepare_svdq_layer(w.astype(np.float64), L.smooth_factors(x, w.astype(np.float64)), 32, precision, b)
    y_ref = F.bf16_to_f32(host_bits(bq.SVDQLinear.from_numpy(lay)(xd))).astype(np.float64)
    e_gpu = np.linalg.norm(y_gpu - exact) / np.linalg.norm(exact)
    e_ref = np.linalg.norm(y_ref - exact) / np.linalg.norm(exact)
    print(f"[prepare {precision}] relative error: GPU-prepared {e_gpu:.4e}, oracle-prepared {e_ref:.4e}", flush=True)
    assert e_gpu <= 1.05 * e_ref
