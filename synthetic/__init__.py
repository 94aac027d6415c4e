"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and casts them to bfloat16 with torch; it
holds none of the quantization method's arithmetic (no scales, no codes, no
smoothing, no SVD).  The workloads stand in for the DiT layers of the Nunchaku
Lite pages (ERNIE-Image-Turbo / Flux transformers at 1024x1024), whose trained
checkpoints are not available: activations are N(0, 1) with a few outlier
channels scaled by 20, weights N(0, 0.02) with a rank-8 spike.

Every tensor gets its own stream spawned from ``numpy.random.SeedSequence(seed)``.
bfloat16 tensors are returned as uint16 bit patterns (numpy).
"""

import math

import numpy as np
import torch


def streams(seed, n):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def to_bf16_bits(a):
    """float array -> bfloat16 bit patterns (uint16), via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_float(b):
    """bfloat16 bit patterns -> float32 values, via torch."""
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


def activations(M, K, n_outliers, rng, outlier_scale=20.0):
    """X ~ N(0, 1) [M, K] with ``n_outliers`` channels scaled by ``outlier_scale``."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_outliers:
        cols = rng.choice(K, n_outliers, replace=False)
        x[:, cols] *= outlier_scale
    return to_bf16_bits(x)


def weight(N, K, std, rng, spike_rank=0, spike_factor=5.0):
    """W ~ N(0, std) [N, K] plus an optional low-rank spike, as bf16 values (float64).

    The spike adds ``spike_rank`` components with random orthonormal singular
    vectors, each of singular value spike_factor * std * (sqrt(N) + sqrt(K)),
    i.e. ``spike_factor`` times the largest singular value a Gaussian matrix
    of that size has (the Marchenko-Pastur edge).
    """
    w = rng.standard_normal((N, K)) * std
    if spike_rank:
        u, _ = np.linalg.qr(rng.standard_normal((N, spike_rank)))
        v, _ = np.linalg.qr(rng.standard_normal((K, spike_rank)))
        sv = spike_factor * std * (math.sqrt(N) + math.sqrt(K))
        w = w + (u * sv) @ v.T
    return bits_to_float(to_bf16_bits(w)).astype(np.float64)


def bias(N, rng, std=0.01):
    return to_bf16_bits(rng.standard_normal(N) * std)


def rope_tables(M, D, base=10000.0, offset=0):
    """Rotary-embedding angle tables for M tokens at positions offset ..
    offset + M - 1 and head dim D: angle[m, i] = pos_m * base^(-2i/D),
    returned as float32 (cos, sin) [M, D/2].  The model's positional input,
    not part of the layer."""
    pos = np.arange(offset, offset + M, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)[None, :]
    ang = pos * inv
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def norm_weight(D, rng):
    """A learned RMSNorm weight [D] as bf16 bits, around 1."""
    return to_bf16_bits(1.0 + 0.1 * rng.standard_normal(D))


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
CONFIG_NAMES = {
    0: "tiny svdq_w4a4 int4 64x256x256",
    1: "svdq_w4a4 int4 M=4096 K=N=3072 (DiT attention projection)",
    2: "svdq_w4a4 nvfp4 M=4096 K=N=3072 + MLP 3072->12288->3072",
    3: "awq_w4a16 int4 M in {1,2,16}, K=3072, N=18432 (adaLN modulation)",
    4: "DiT stack: 24 blocks x (QKV, out, MLP up/down svdq nvfp4 r32; adaLN awq M=1), 4096 tokens",
}


def svdq_problem(M, K, N, seed, n_outliers, spike_rank=8, std=0.02, with_bias=True):
    """Inputs of one svdq_w4a4 linear: X bf16 bits, W float64, bias bits."""
    rx, rw, rb = streams(seed, 3)
    x = activations(M, K, n_outliers, rx)
    w = weight(N, K, std, rw, spike_rank=spike_rank)
    b = bias(N, rb) if with_bias else None
    return x, w, b


def config0(seed=0):
    """Tiny int4 case: X [64, 256] with 4 outlier channels, W [256, 256] N(0, 0.02)
    (no spike), smooth = ones, rank 32, group 64."""
    x, w, b = svdq_problem(64, 256, 256, seed, n_outliers=4, spike_rank=0)
    return dict(x=x, w=w, bias=b, precision="int4", rank=32, smooth="ones")


def config1(seed=0, M=4096, K=3072, N=3072):
    """int4 DiT projection: 1 % of channels (31 of 3072) are outliers, rank-8 spike,
    smoothing calibrated on X."""
    x, w, b = svdq_problem(M, K, N, seed, n_outliers=round(0.01 * K))
    return dict(x=x, w=w, bias=b, precision="int4", rank=32, smooth="calibrated")


def config2(seed=0, M=4096, K=3072, N=3072, hidden=12288):
    """nvfp4 projection (same recipe as config 1) plus the MLP pair
    up K->hidden and down hidden->K (the down input is GELU of the up output)."""
    proj = config1(seed, M, K, N)
    proj["precision"] = "nvfp4"
    rw1, rw2, rb1, rb2 = streams(seed + 1000, 4)
    w_up = weight(hidden, K, 0.02, rw1, spike_rank=8)
    w_down = weight(K, hidden, 0.02, rw2, spike_rank=8)
    return dict(proj=proj, w_up=w_up, b_up=bias(hidden, rb1), w_down=w_down,
                b_down=bias(K, rb2), precision="nvfp4", rank=32)


def config3(seed=0, Ms=(1, 2, 16), K=3072, N=18432):
    """AWQ adaLN modulation linears: X [M, K] N(0, 1) for each M, W [N, K] N(0, 0.02)."""
    rw, rb, *rxs = streams(seed, 2 + len(Ms))
    w = weight(N, K, 0.02, rw)
    xs = {M: activations(M, K, 0, r) for M, r in zip(Ms, rxs)}
    return dict(w=w, bias=bias(N, rb), xs=xs)


STACK_LAYERS = (("qkv", 3072, 9216), ("out", 3072, 3072), ("up", 3072, 12288),
                ("down", 12288, 3072))
STACK = dict(blocks=24, tokens=4096, hidden=3072, adaln=(3072, 18432), passes=8, rank=32)


# ----------------------------------------------------------------------------
# random-valid packed layers (for timing: the values of prepared weights do
# not change the work a call does)
# ----------------------------------------------------------------------------
def random_svdq_layer(N, K, precision, rank, rng, device=None):
    """Random but valid inputs of svdq_w4a4_linear for a [N, K] layer.

    int4: sign-magnitude nibbles with magnitude <= 7 (every nibble is legal),
    bf16 group scales ~ 1e-3..1e-2; nvfp4: any nibble (E2M1), E4M3 scale codes
    drawn from the normal range, tensor scale 2^-7.  smooth in [0.5, 2],
    lora factors N(0, 0.02), bias N(0, 0.01).  Returns numpy arrays.
    """
    G = 64 if precision == "int4" else 16
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    if precision == "int4":
        wscales = to_bf16_bits(rng.uniform(1e-3, 1e-2, size=(N, K // G)))
        wt = 1.0
    else:
        wscales = rng.integers(0x30, 0x60, size=(N, K // G), dtype=np.uint8)
        wt = 2.0 ** -7
    smooth = to_bf16_bits(rng.uniform(0.5, 2.0, size=K))
    down = to_bf16_bits(rng.standard_normal((rank, K)) * 0.02)
    up = to_bf16_bits(rng.standard_normal((N, rank)) * 0.02)
    b = to_bf16_bits(rng.standard_normal(N) * 0.01)
    return dict(packed_w=packed, wscales=wscales, wtscale=wt, smooth=smooth,
                lora_down=down, lora_up=up, bias=b, precision=precision,
                group_size=G, rank=rank, N=N, K=K)


def random_awq_layer(N, K, rng, G=64):
    """Random valid awq_w4a16 inputs: uint4 codes, bf16 scales ~1e-3..1e-2,
    integer zero-points 0..15 stored as bf16, bias N(0, 0.01)."""
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = to_bf16_bits(rng.uniform(1e-3, 1e-2, size=(N, K // G)))
    z = to_bf16_bits(rng.integers(0, 16, size=(N, K // G)).astype(np.float32))
    b = to_bf16_bits(rng.standard_normal(N) * 0.01)
    return dict(packed_w=packed, wscales=s, wzeros=z, bias=b, group_size=G, N=N, K=K)
