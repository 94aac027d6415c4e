"""Activation inputs that put the quantizer on exact rounding ties.

Each function returns (x bf16 bits [M, K], smooth bf16 bits [K], cases), where
``cases`` lists (row, group) positions of the constructed ties so that tests
can assert they are ties before using them.  The ties (all decided by round
half to even):

* int4 codes: a group with amax 7 * 2^e has scale s = 2^e exactly, and the
  values (n + 1/2) 2^e give x / s = n + 1/2 for n = 0..6, both signs;
* int4 scales: none exist -- fl32(amax / 7) is never halfway between two
  bfloat16 values when x and smooth are bfloat16 (int4_scale_tie_count
  enumerates every case; see its docstring);
* nvfp4 scales: amax / 6 exactly halfway between two E4M3 values, for every
  pair of neighbours from 0 up to 448, and at the 448 / 464 saturation edge;
* nvfp4 codes: a group with amax 6 * 2^e has S = 2^e, and the values m 2^e
  for every E2M1 midpoint m in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}.

Only numpy float32 arithmetic and the bfloat16 cast of ``synthetic`` are used
to build them; the expected codes come from the oracle in the tests.
"""

import numpy as np

import synthetic as S

F32 = np.float32


def _bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(F32)


def int4_code_ties(exps=(-30, -20, -17, -10, -3, 0, 3, 10, 12, 13, 20), groups_per_row=4):
    """Rows of int4 groups with exact code ties; each row's groups share one
    exponent (rows with 2^e outside [2^-17, 2^13) take the rewritten operand
    path), plus rows mixing two far-apart exponents."""
    half = [(n + 0.5) for n in range(7)]
    pattern = [7.0] + half + [-h for h in half] + [float(v) for v in range(-7, 8)]
    pattern = (pattern * 3)[:64]
    rows, cases = [], []
    for e in exps:
        rows.append(np.tile(np.array(pattern) * 2.0 ** e, groups_per_row))
    rows.append(np.concatenate([np.array(pattern) * 2.0 ** e for e in (-20, 0, 10, -3)]))
    rows.append(np.concatenate([np.array(pattern) * 2.0 ** e for e in (14, -17, 1, -16)]))
    x = np.array(rows)
    for r in range(x.shape[0]):
        for g in range(groups_per_row):
            cases.append((r, g))
    xb = S.to_bf16_bits(x)
    assert np.array_equal(_bits_to_f32(xb).astype(np.float64), x), "tie values must be exact bf16"
    return xb, S.to_bf16_bits(np.ones(x.shape[1], np.float32)), cases


def int4_scale_tie_count():
    """Number of bf16 (x, smooth) pairs whose int4 group scale would be a
    bfloat16 rounding tie, i.e. fl32(fl32(x * fl32(1 / smooth)) / 7) has its
    low 16 bits equal to 0x8000 (exactly halfway between two bfloat16
    values), with x the group's largest magnitude.

    Multiplying x or smooth by a power of two scales every intermediate by
    the same power of two (exactly, in the normal range), so only the 128
    significands 1.xxxxxxx of each matter, and all 128 x 128 pairs are
    enumerated.  (Why the count is 0: the quotient rounds to a 9-bit value
    only if x_hat = 7 q exactly, a 12-bit significand, but x_hat has at most
    8 significant bits when 1/smooth is exact and at least 16 otherwise.)"""
    sig = _bits_to_f32(np.arange(0x3F80, 0x4000, dtype=np.uint16))  # [1, 2)
    mu = (F32(1.0) / sig).astype(F32)
    xh = (sig[:, None] * mu[None, :]).astype(F32)
    q = (xh / F32(7.0)).astype(F32)
    return int(np.sum((q.view(np.uint32) & 0xFFFF) == 0x8000))


def e4m3_midpoints():
    """Every midpoint between neighbouring non-negative E4M3 values up to 448,
    and the saturation edge (464 = 448 + half a step, 456, 480)."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(-6, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** e
            if v <= 448:
                vals.append(v)
    vals = np.array(sorted(vals))
    mids = (vals[1:] + vals[:-1]) / 2
    return np.concatenate([mids, [456.0, 464.0, 480.0]])


def nvfp4_scale_ties(K=256, seed=1):
    """One group per E4M3 midpoint m: amax = 6 m exactly (so fl32(amax / 6)
    is m), the other 15 values below it; several groups per row."""
    rng = np.random.default_rng(seed)
    mids = e4m3_midpoints()
    per_row = K // 16
    n_rows = -(-len(mids) // per_row)
    x = np.zeros((n_rows, K), np.float64)
    cases = []
    for i, m in enumerate(mids):
        r, g = divmod(i, per_row)
        vals = rng.uniform(-0.95, 0.95, 16) * 6 * m
        vals[i % 16] = 6 * m if i % 2 == 0 else -6 * m
        x[r, 16 * g:16 * g + 16] = vals
        cases.append((r, g))
    xb = S.to_bf16_bits(x)
    xf = _bits_to_f32(xb).astype(np.float64)
    for (r, g), m in zip(cases, mids):
        assert np.abs(xf[r, 16 * g:16 * g + 16]).max() == 6 * m, "amax must be exactly 6 m"
    return xb, S.to_bf16_bits(np.ones(K, np.float32)), cases


def nvfp4_code_ties(exps=(-9, -5, -1, 0, 2, 5, 8), K=256):
    """Groups with amax 6 * 2^e (S = 2^e) holding every E2M1 midpoint times
    2^e, both signs."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    pattern = np.array([6.0] + mids + [-m for m in mids] + [-6.0])
    rows = [np.tile(pattern * 2.0 ** e, K // 16) for e in exps]
    x = np.array(rows)
    xb = S.to_bf16_bits(x)
    assert np.array_equal(_bits_to_f32(xb).astype(np.float64), x)
    cases = [(r, g) for r in range(len(exps)) for g in range(K // 16)]
    return xb, S.to_bf16_bits(np.ones(K, np.float32)), cases
