"""The fused MLP's bf16 GELU table, against the oracle's bf16 GELU on every
finite bf16 input.

CPU: the build-time generator (double-precision erfc from the C library,
one rounding to bf16) -- an implementation independent of the oracle's
(scipy's erfc).  GPU: the table as compiled into the library, read back
through its parity export.
"""

import numpy as np
import pytest

from oracle import formats as F, layers as L

bq = pytest.importorskip("bit_quantized_linear_quantize_amd")


def _finite_bits():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return bits, np.isfinite(F.bf16_to_f32(bits))


def test_generator_matches_oracle_exhaustively():
    from bit_quantized_linear_quantize_amd import gelu_bf16_gen as gelu_table
    bits, fin = _finite_bits()
    got = np.array(gelu_table.table(), dtype=np.uint16)
    want = L.gelu_bf16(bits[fin])
    bad = np.nonzero(got[fin] != want)[0]
    assert bad.size == 0, [(int(bits[fin][i]), int(got[fin][i]), int(want[i])) for i in bad[:8]]
    # non-finite inputs: +inf -> +inf, -inf and NaN -> NaN
    assert got[0x7F80] == 0x7F80
    assert np.isnan(F.bf16_to_f32(got[[0xFF80, 0x7FC0, 0xFFC1]])).all()


def test_generator_rounding_edges():
    from bit_quantized_linear_quantize_amd import gelu_bf16_gen as G
    # ties to even, carry into the next binade, subnormals, overflow, signed zero
    assert G.bf16_rne_bits(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (down)
    assert G.bf16_rne_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (up)
    assert G.bf16_rne_bits(2.0 - 2.0 ** -9) == 0x4000          # carry into 2.0
    assert G.bf16_rne_bits(2.0 ** -133) == 0x0001
    assert G.bf16_rne_bits(2.0 ** -134) == 0x0000               # tie -> even zero
    assert G.bf16_rne_bits(3 * 2.0 ** -134) == 0x0002
    assert G.bf16_rne_bits(-0.0) == 0x8000
    assert G.bf16_rne_bits(3.5e38) == 0x7F80
    assert G.bf16_rne_bits(127.5 * 2.0 ** -133) == 0x0080     # tie -> even: the smallest normal
    assert G.bf16_rne_bits(126.5 * 2.0 ** -133) == 0x007E     # tie -> even subnormal


@pytest.mark.gpu
def test_device_table_matches_oracle_exhaustively():
    import torch
    t = bq.gelu_table()
    torch.cuda.synchronize()
    got = t.cpu().numpy().view(np.uint16)
    bits, fin = _finite_bits()
    want = L.gelu_bf16(bits[fin])
    bad = np.nonzero(got[fin] != want)[0]
    assert bad.size == 0, [(int(bits[fin][i]), int(got[fin][i]), int(want[i])) for i in bad[:8]]
