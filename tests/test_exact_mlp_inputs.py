"""Pins of the exact-arithmetic inputs the fused MLP parity tests use: the
oracle's packer and activation quantizer reproduce the constructed values,
every term of the up projection is a multiple of 2^-13 with magnitudes
summing below 2^24 such units, and a float32 accumulation in a shuffled
order gives the oracle's fp64 value exactly."""

import numpy as np
import pytest

from exact_mlp import exact_up_problem
from oracle import formats as F, layers as L


@pytest.mark.parametrize("precision", ["nvfp4", "int4"])
@pytest.mark.parametrize("K,rank", [(256, 0), (256, 128), (3072, 32)])
def test_exact_up_problem(precision, K, rank):
    rng = np.random.default_rng(K + rank)
    M, H = 12, 96
    x, lay = exact_up_problem(M, K, H, precision, rank, rng)
    w = lay["exact_w"]
    assert np.array_equal(L.dequant(lay["w_codes"], lay["wscales"], precision) * lay["wtscale"], w)
    act = L.svdq_quantize_act(x, lay["smooth"], lay["lora_down"], precision)
    xf = F.bf16_to_f32(x).astype(np.float64)
    assert np.array_equal(L.dequant(act["codes"], act["scales"], precision), xf)

    terms = [xf[:, None, :] * w[None, :, :]]
    if rank:
        ld = F.bf16_to_f32(lay["lora_down"]).astype(np.float64)
        lu = F.bf16_to_f32(lay["lora_up"]).astype(np.float64)
        la = xf @ ld.T
        assert np.array_equal(la * 2.0 ** 7, np.round(la * 2.0 ** 7)) and np.abs(la).max() < 2.0 ** 9
        terms.append(la[:, None, :] * lu[None, :, :])
    bias = F.bf16_to_f32(lay["bias"]).astype(np.float64)
    terms.append(np.broadcast_to(bias[None, :, None], (M, H, 1)))
    t = np.concatenate(terms, axis=2)
    u = t * 2.0 ** 13
    assert np.array_equal(u, np.round(u))
    assert np.abs(u).sum(axis=2).max() < 2.0 ** 24

    h = L.svdq_linear_ref(x, lay)
    assert 1.5 < h.std() < 6.0
    acc = np.zeros((M, H), np.float32)
    for j in rng.permutation(t.shape[2]):
        acc += t[:, :, j].astype(np.float32)
    assert np.array_equal(acc.astype(np.float64), h)
