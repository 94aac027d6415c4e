"""The documented split-K rule of svdq_w4a4_linear (include/svdq_w4a4.h, and
the workspace layout it implies), restated for the tests."""


def ksplit(M, N, K):
    """Split only when the 256 x 192 output tiles fill less than half of 256
    compute units; up to 8 splits of at least 2 64-column stages, every split
    non-empty."""
    tiles = -(-M // 256) * -(-N // 192)
    nst = K // 64
    if tiles >= 128:
        return 1
    s = max(min(8, 256 // tiles, nst // 2), 1)
    while s > 1 and -(-nst // s) * (s - 1) >= nst:
        s -= 1
    return s


def split_bytes(M, N, K):
    s = ksplit(M, N, K)
    return 0 if s == 1 else (s * M * N * 4 + 255) // 256 * 256
