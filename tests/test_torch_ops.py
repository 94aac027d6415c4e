"""The two linears as torch.library custom ops.

CPU: the ops are registered and trace through their fake implementations.
GPU: through the custom ops the outputs equal the plain binding's bit for bit
and meet the oracle bar; torch.library.opcheck passes; a function calling
both ops compiles with torch.compile(fullgraph=True) and gives the same bits.
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F, layers as L

bq = pytest.importorskip("bit_quantized_linear_quantize_amd")
from bit_quantized_linear_quantize_amd import torch_ops as T  # noqa: E402


def _fake_args():
    bf, u8 = torch.bfloat16, torch.uint8
    M, K, N, r, Na = 64, 256, 320, 32, 128
    return (torch.zeros(M, K, dtype=bf), torch.zeros(N, K // 2, dtype=u8), torch.zeros(N, K // 64, dtype=bf),
            torch.zeros(K, dtype=bf), torch.zeros(r, K, dtype=bf), torch.zeros(N, r, dtype=bf),
            torch.zeros(N, dtype=bf), torch.zeros(Na, N // 2, dtype=u8), torch.zeros(Na, N // 64, dtype=bf),
            torch.zeros(Na, N // 64, dtype=bf))


def _pair(x, pw, ws, sm, ld, lu, b, apw, aws, awz):
    h = torch.ops.svdq.w4a4_linear(x, pw, ws, 1.0, sm, ld, lu, b, "int4")
    return torch.ops.svdq.awq_w4a16_linear(h, apw, aws, awz, None)


def test_ops_trace_on_fake_tensors():
    from torch.fx.experimental.proxy_tensor import make_fx
    g = make_fx(_pair, tracing_mode="fake")(*_fake_args())
    targets = [n.target for n in g.graph.nodes if n.op == "call_function"]
    assert torch.ops.svdq.w4a4_linear.default in targets
    assert torch.ops.svdq.awq_w4a16_linear.default in targets
    out = [n for n in g.graph.nodes if n.op == "output"][0].args[0]
    meta = out[0].meta["val"] if isinstance(out, (tuple, list)) else out.meta["val"]
    assert tuple(meta.shape) == (64, 128) and meta.dtype == torch.bfloat16


# ------------------------------------------------------------------ GPU
def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def layers():
    rng = np.random.default_rng(21)
    M, K, N, Na = 96, 512, 384, 256
    x = S.activations(M, K, 5, rng)
    w = S.weight(N, K, 0.02, rng, spike_rank=2)
    lay = L.prepare_svdq_layer(w, L.smooth_factors(x, w), 32, "int4", S.bias(N, rng))
    wa = rng.standard_normal((Na, N)) * 0.02
    alay = L.prepare_awq_layer(wa, S.bias(Na, rng))
    xa = S.activations(M, N, 3, rng)
    return x, lay, alay, xa


@pytest.mark.gpu
def test_custom_ops_match_binding_and_oracle(layers):
    x, lay, alay, xa = layers
    layer, alayer = bq.SVDQLinear.from_numpy(lay), bq.AWQLinear.from_numpy(alay)
    xd, xad = dev_bf16(x), dev_bf16(xa)
    y_op = T.svdq_linear(xd, layer)
    y_b = bq.svdq_w4a4_linear(xd, layer)
    h_op = T.awq_linear(xad, alayer)
    h_b = bq.awq_w4a16_linear(xad, alayer)
    # chained, as a model calls them
    c_op = T.awq_linear(y_op, alayer)
    c_b = bq.awq_w4a16_linear(y_b, alayer)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y_op), host_bits(y_b))
    assert np.array_equal(host_bits(h_op), host_bits(h_b))
    assert np.array_equal(host_bits(c_op), host_bits(c_b))
    y = F.bf16_to_f32(host_bits(y_op)).astype(np.float64)
    _, excess, mre = L.output_errors(y, L.svdq_linear_ref(x, lay))
    assert excess <= 1e-2 and mre <= 2e-3
    h = F.bf16_to_f32(host_bits(h_op)).astype(np.float64)
    _, excess, mre = L.output_errors(h, L.awq_linear_ref(xa, alay))
    assert excess <= 1e-2 and mre <= 2e-3


@pytest.mark.gpu
def test_custom_ops_opcheck(layers):
    x, lay, alay, _ = layers
    layer, alayer = bq.SVDQLinear.from_numpy(lay), bq.AWQLinear.from_numpy(alay)
    xd = dev_bf16(x)
    torch.library.opcheck(torch.ops.svdq.w4a4_linear.default,
                          (xd, layer.packed_w, layer.wscales, layer.wtscale, layer.smooth, layer.lora_down,
                           layer.lora_up, layer.bias, layer.precision))
    h = bq.svdq_w4a4_linear(xd, layer)
    torch.library.opcheck(torch.ops.svdq.awq_w4a16_linear.default,
                          (h, alayer.packed_w, alayer.wscales, alayer.wzeros, alayer.bias))


@pytest.mark.gpu
@pytest.mark.parametrize("backend", ["aot_eager", "inductor"])
def test_compile_fullgraph(layers, backend):
    # an elementwise op between the two linears, which Inductor generates itself
    x, lay, alay, _ = layers
    layer, alayer = bq.SVDQLinear.from_numpy(lay), bq.AWQLinear.from_numpy(alay)
    xd = dev_bf16(x)

    def f(inp):
        return T.awq_linear(T.svdq_linear(inp, layer) * 0.5, alayer)

    ref = f(xd)
    got = torch.compile(f, fullgraph=True, backend=backend)(xd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(got), host_bits(ref))


# ------------------------------------------------------------------ the fused entry points
def _fake_fused_args():
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    M, K, H, N, r, heads = 64, 256, 640, 256, 32, 2
    up = (torch.zeros(H, K // 2, dtype=u8), torch.zeros(H, K // 16, dtype=u8), 1.0, torch.zeros(K, dtype=bf),
          torch.zeros(r, K, dtype=bf), torch.zeros(H, r, dtype=bf), torch.zeros(H, dtype=bf))
    dn = (torch.zeros(N, H // 2, dtype=u8), torch.zeros(N, H // 16, dtype=u8), 1.0, torch.zeros(H, dtype=bf),
          torch.zeros(r, H, dtype=bf), torch.zeros(N, r, dtype=bf), torch.zeros(N, dtype=bf))
    Nq = 3 * heads * 128
    qkv = (torch.zeros(Nq, K // 2, dtype=u8), torch.zeros(Nq, K // 16, dtype=u8), 1.0, torch.zeros(K, dtype=bf),
           torch.zeros(r, K, dtype=bf), torch.zeros(Nq, r, dtype=bf), torch.zeros(Nq, dtype=bf))
    norms = (torch.zeros(128, dtype=bf), torch.zeros(128, dtype=bf), torch.zeros(M, 64, dtype=f32),
             torch.zeros(M, 64, dtype=f32))
    return torch.zeros(M, K, dtype=bf), up, dn, qkv, heads, norms


def test_fused_ops_trace_on_fake_tensors():
    from torch.fx.experimental.proxy_tensor import make_fx
    x, up, dn, qkv, heads, norms = _fake_fused_args()
    tensors = [a for a in up + dn + qkv + norms if isinstance(a, torch.Tensor)]

    def f(x, *t):
        it = iter(t)
        take = lambda args: tuple(next(it) if isinstance(a, torch.Tensor) else a for a in args)
        u, d, q, n = take(up), take(dn), take(qkv), take(norms)
        y = torch.ops.svdq.w4a4_mlp_gelu(x, *u, "nvfp4", *d)
        z = torch.ops.svdq.w4a4_qkv_rmsnorm_rope(x, *q, "nvfp4", heads, *n, 1e-6)
        return y, z
    g = make_fx(f, tracing_mode="fake")(x, *tensors)
    targets = [n.target for n in g.graph.nodes if n.op == "call_function"]
    assert torch.ops.svdq.w4a4_mlp_gelu.default in targets
    assert torch.ops.svdq.w4a4_qkv_rmsnorm_rope.default in targets
    outs = [n for n in g.graph.nodes if n.op == "output"][0].args[0]
    assert tuple(outs[0].meta["val"].shape) == (64, 256) and tuple(outs[1].meta["val"].shape) == (64, 768)


@pytest.fixture(scope="module")
def fused_layers():
    from exact_mlp import exact_up_problem
    rng = np.random.default_rng(33)
    M, K, H, N, heads = 96, 256, 640, 256, 2
    x, up = exact_up_problem(M, K, H, "nvfp4", 32, rng)
    h = F.bf16_bits_f64(L.svdq_linear_ref(x, up))
    w_dn = S.weight(N, H, 0.02, rng)
    down = L.prepare_svdq_layer(w_dn, L.smooth_factors(L.gelu_bf16(h), w_dn), 32, "nvfp4", S.bias(N, rng))
    qkv = L.prepare_svdq_layer(S.weight(3 * heads * 128, K, 0.05, rng), np.full(K, 0x3F80, np.uint16), 32, "nvfp4",
                               S.bias(3 * heads * 128, rng))
    qn, kn = S.norm_weight(128, rng), S.norm_weight(128, rng)
    cos, sin = S.rope_tables(M, 128)
    return x, up, down, qkv, heads, qn, kn, cos, sin


def _dev_norms(qn, kn, cos, sin):
    return dev_bf16(qn), dev_bf16(kn), torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()


@pytest.mark.gpu
def test_fused_custom_ops_match_binding(fused_layers):
    x, up, down, qkv, heads, qn, kn, cos, sin = fused_layers
    U, D, Q = (bq.SVDQLinear.from_numpy(a) for a in (up, down, qkv))
    xd = dev_bf16(x)
    norms = _dev_norms(qn, kn, cos, sin)
    q_op = T.qkv_rmsnorm_rope(xd, Q, heads, *norms)
    q_b = bq.svdq_w4a4_qkv_rmsnorm_rope(xd, Q, heads, *norms)
    y_op = T.mlp_gelu(xd, U, D)
    y_b = bq.svdq_w4a4_mlp_gelu(xd, U, D)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(q_op), host_bits(q_b))
    # (the MLP's low-rank accumulation uses fp32 atomics: last bits may vary)
    a = F.bf16_to_f32(host_bits(y_op)).astype(np.float64)
    b = F.bf16_to_f32(host_bits(y_b)).astype(np.float64)
    _, excess, mre = L.output_errors(a, b)
    assert excess <= 1e-3 and mre <= 1e-3


@pytest.mark.gpu
def test_fused_custom_ops_opcheck(fused_layers):
    x, up, down, qkv, heads, qn, kn, cos, sin = fused_layers
    U, D, Q = (bq.SVDQLinear.from_numpy(a) for a in (up, down, qkv))
    xd = dev_bf16(x)
    la = lambda l: (l.packed_w, l.wscales, l.wtscale, l.smooth, l.lora_down, l.lora_up, l.bias)
    torch.library.opcheck(torch.ops.svdq.w4a4_qkv_rmsnorm_rope.default,
                          (xd, *la(Q), Q.precision, heads, *_dev_norms(qn, kn, cos, sin), 1e-6))
    torch.library.opcheck(torch.ops.svdq.w4a4_mlp_gelu.default, (xd, *la(U), U.precision, *la(D)))


@pytest.mark.gpu
@pytest.mark.parametrize("backend", ["aot_eager", "inductor"])
def test_fused_compile_fullgraph(fused_layers, backend):
    x, up, down, qkv, heads, qn, kn, cos, sin = fused_layers
    U, D, Q = (bq.SVDQLinear.from_numpy(a) for a in (up, down, qkv))
    xd = dev_bf16(x)
    norms = _dev_norms(qn, kn, cos, sin)

    def f(inp):
        return T.qkv_rmsnorm_rope(inp * 1.0, Q, heads, *norms), T.mlp_gelu(inp, U, D)
    ref_q, ref_y = f(xd)
    got_q, got_y = torch.compile(f, fullgraph=True, backend=backend)(xd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(got_q), host_bits(ref_q))
    # the fused MLP is deterministic: the compiled call gives the eager bits
    assert np.array_equal(host_bits(got_y), host_bits(ref_y))
