"""The documented split-K rule of svdq_w4a4_linear (include/svdq_w4a4.h, and
the workspace layout it implies), restated for the tests."""


def ksplit(M, N, K, precision="nvfp4"):
    """Split only when the 256 x 192 output tiles fill at most half of 256
    compute units; up to 8 splits of at least 2 stages (128 values of K for
    int4, 64 for nvfp4) and at most max(2, stages // 5) splits, every split
    non-empty."""
    tiles = -(-M // 256) * -(-N // 192)
    nst = K // (128 if precision in ("int4", 0) else 64)
    if tiles > 128:
        return 1
    s = max(min(8, 256 // tiles, nst // 2, max(2, nst // 5)), 1)
    while s > 1 and -(-nst // s) * (s - 1) >= nst:
        s -= 1
    return s


def split_bytes(M, N, K, precision="nvfp4"):
    s = ksplit(M, N, K, precision)
    return 0 if s == 1 else (s * M * N * 4 + 255) // 256 * 256


def k1_slices(M, K):
    """Kernel 1 of the linear splits K over S workgroups per 16 rows (1, 2, 4
    or 8, dividing the K/64 chunks) while the row blocks alone would leave
    more than half of 256 compute units idle."""
    blocks, chunks, s = -(-M // 16), K // 64, 1
    while s < 8 and blocks * s * 2 <= 256 and chunks % (s * 2) == 0:
        s *= 2
    return s


def lora_part_bytes(M, K, rank):
    """The workspace part holding kernel 1's low-rank slice partials."""
    s = k1_slices(M, K)
    return 0 if s == 1 else (s * M * rank * 4 + 255) // 256 * 256
