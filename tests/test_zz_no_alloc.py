"""svdq_w4a4_linear_noalloc (the allocation-free linear: static device
scratch instead of a workspace) against svdq_w4a4_linear through the C ABI:
bit-identical outputs on consecutive calls that share the scratch -- the
second call smaller than the first -- and a clear error, with nothing
written, for a call whose scratch need exceeds the static array."""

import numpy as np
import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_linear_quantize_amd")


def layer_and_x(M, K, N, precision, rank, seed):
    rl, rx = S.streams(seed, 2)
    layer = bq.SVDQLinear.from_numpy(S.random_svdq_layer(N, K, precision, rank, rl))
    x = torch.from_numpy(S.activations(M, K, round(0.01 * K), rx).view(np.int16).copy()).view(torch.bfloat16).cuda()
    return layer, x


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def test_noalloc_matches_linear_on_consecutive_calls():
    # largest first: config 1 (25.7 MB of scratch), then one GPU's token
    # share of it (M = 512: the product split along K, 27.4 MB), then a
    # small ragged call; each must equal the workspace entry point bit for bit
    cases = [(4096, 3072, 3072, "int4", 32), (512, 3072, 3072, "int4", 32), (300, 512, 320, "nvfp4", 16),
             (37, 256, 192, "int4", 0)]
    for i, (M, K, N, p, r) in enumerate(cases):
        layer, x = layer_and_x(M, K, N, p, r, seed=100 + i)
        need = layer.workspace_bytes(M)
        assert need <= bq.NOALLOC_SCRATCH_BYTES
        ref = layer(x)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        bq.svdq_w4a4_linear_noalloc(x, layer, out)
        torch.cuda.synchronize()
        print(f"[noalloc M={M} K={K} N={N} {p} r{r}] scratch {need} bytes", flush=True)
        assert np.array_equal(bits(out), bits(ref)), (M, K, N, p, r)


def test_noalloc_rejects_oversize_without_writing():
    # M = 16384, K = 3072, N = 64 (split K): 69.7 MB of scratch, more than the static 64 MiB
    M, K, N = 16384, 3072, 64
    layer, x = layer_and_x(M, K, N, "int4", 16, seed=7)
    assert layer.workspace_bytes(M) > bq.NOALLOC_SCRATCH_BYTES
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bq.SvdqError) as e:
        bq.svdq_w4a4_linear_noalloc(x, layer, out)
    assert e.value.status == -4 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))
