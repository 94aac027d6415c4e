"""The tie constructions of tests/tie_inputs.py really are ties (CPU), and the
int4 activation scale has no bfloat16 ties to construct."""

import numpy as np

import tie_inputs as T
from oracle import formats as F, layers as L


def test_int4_scale_has_no_bf16_ties():
    assert T.int4_scale_tie_count() == 0


def test_int4_code_ties_are_ties():
    x, sm, cases = T.int4_code_ties()
    xh = L.smoothed_activations(x, sm).astype(np.float64)
    for r, g in cases:
        grp = xh[r, 64 * g:64 * g + 64]
        s = np.abs(grp).max() / 7
        assert s == 2.0 ** np.floor(np.log2(s))            # s = 2^e exactly
        t = grp / s
        assert {n + 0.5 for n in range(7)} | {-n - 0.5 for n in range(7)} <= set(t)   # every n + 1/2, both signs


def test_nvfp4_scale_ties_are_ties():
    x, sm, cases = T.nvfp4_scale_ties()
    xh = L.smoothed_activations(x, sm)
    mids = T.e4m3_midpoints()
    for (r, g), m in zip(cases, mids):
        amax = np.abs(xh[r, 16 * g:16 * g + 16]).max()
        assert np.float32(amax / np.float32(6.0)) == m
    # every in-range midpoint: strictly between two neighbouring E4M3 values
    grid = np.unique(np.abs(F.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)))
    grid = grid[np.isfinite(grid)]
    for m in mids[mids < 448]:
        i = np.searchsorted(grid, m)
        assert grid[i - 1] < m < grid[i] and m - grid[i - 1] == grid[i] - m


def test_nvfp4_code_ties_are_ties():
    x, sm, cases = T.nvfp4_code_ties()
    xh = L.smoothed_activations(x, sm).astype(np.float64)
    mids = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0}
    for r, g in cases:
        grp = xh[r, 16 * g:16 * g + 16]
        S = np.abs(grp).max() / 6
        assert {abs(v) / S for v in grp} >= mids
