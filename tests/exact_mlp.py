"""Inputs on which an svdq_w4a4 up projection is exact in fp32.

The fused GELU MLP computes the up projection's bf16 output h inside one
kernel and quantizes GELU(h) for the down projection.  Where fp32
accumulation and the oracle's fp64 differ in the last bits, bf16(h) can
differ in the last place, and a 4-bit code of the next layer can follow it.
On the inputs built here every product, every partial sum and the result are
multiples of one power of two (2^-12 or 2^-13) below 2^24 of it, so every
accumulation order gives the same exact value, bf16(h) is unique, and the
oracle alone fixes the whole fused chain.

nvfp4: x holds E2M1 values with one +-6 per 16-group (activation scale 1);
w = code * c_g * 2^-k with E2M1 codes, one +-6 per group, E4M3 group factors
c_g in 8..15 and one group with 448 (so the tensor scale amax / 2688 = 2^-k).
int4: x holds integers in [-7, 7] with one +-7 per 64-group (scale 1);
w = q * c_g * 2^-k with q in [-7, 7], one |q| = 7 per group, c_g in 1..15.
Low rank: lora_down rows with 8 nonzero entries, integers in [-8, 8] times
2^-6; lora_up integers in [-8, 8] times 2^-5.  Bias: multiples of 2^-6.
k is chosen so that h has an RMS near 3 (the range where GELU bends).
Smoothing factors are 1.
"""

import numpy as np

from oracle import formats as F, layers as L

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _signed(vals, shape, rng):
    v = rng.choice(vals, shape)
    return np.where(rng.random(shape) < 0.5, -v, v)


def _pin_group_max(a, G, vmax, rng):
    R, K = a.shape
    g = a.reshape(R, K // G, G).copy()
    pos = rng.integers(0, G, (R, K // G))
    sign = np.where(rng.random((R, K // G)) < 0.5, -1.0, 1.0)
    np.put_along_axis(g, pos[..., None], (sign * vmax)[..., None], axis=2)
    return g.reshape(R, K)


def exact_up_problem(M, K, H, precision, rank, rng):
    """(x bf16 bits [M, K], oracle layer dict [H, K]) as described above."""
    if precision == "nvfp4":
        G = 16
        x = _pin_group_max(_signed(E2M1, (M, K), rng), G, 6.0, rng)
        q = _pin_group_max(_signed(E2M1, (H, K), rng), G, 6.0, rng)
        c = rng.integers(8, 16, (H, K // G)).astype(np.float64)
        c.flat[rng.integers(c.size)] = 448.0
        rms = np.sqrt(K) * 3.0 * 3.0 * 11.5
    else:
        G = 64
        x = _pin_group_max(rng.integers(-7, 8, (M, K)).astype(np.float64), G, 7.0, rng)
        q = _pin_group_max(rng.integers(-7, 8, (H, K)).astype(np.float64), G, 7.0, rng)
        c = rng.integers(1, 16, (H, K // G)).astype(np.float64)
        rms = np.sqrt(K) * 4.3 * 4.3 * 9.1
    k = int(np.round(np.log2(rms / 3.0)))
    w = (q.reshape(H, K // G, G) * c[..., None]).reshape(H, K) * 2.0 ** -k
    bias = np.round(rng.standard_normal(H) * 0.5 * 64.0) / 64.0
    ones = np.full(K, 0x3F80, np.uint16)
    lay = L.prepare_svdq_layer(w, ones, 0, precision, F.bf16_bits_f64(bias))
    if rank:
        ld = np.zeros((rank, K))
        for r in range(rank):
            ld[r, rng.choice(K, 8, replace=False)] = rng.integers(-8, 9, 8) * 2.0 ** -6
        lu = rng.integers(-8, 9, (H, rank)) * 2.0 ** -5
        lay.update(rank=rank, lora_down=F.bf16_bits_f64(ld), lora_up=F.bf16_bits_f64(lu))
    lay["exact_w"] = w
    return F.bf16_bits_f64(x), lay

