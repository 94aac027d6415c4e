"""The Python binding checks every tensor's dtype, shape and contiguity before
a pointer reaches the C ABI (which trusts the sizes it is given), so a
caller's mistake raises ValueError instead of reaching device memory.

CPU only: with correctly shaped CPU tensors the binding stops at its last
check ("must be a CUDA tensor"); every mismatch below must be reported before
that, by name."""

import pytest
import torch

import bit_quantized_linear_quantize_amd as bq

BF, U8, F32 = torch.bfloat16, torch.uint8, torch.float32


def t(shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


class FakeLayer:
    """The attributes svdq entry points read from an SVDQLinear, on the CPU."""

    def __init__(self, K=256, N=192, rank=16, precision="int4"):
        G = bq.GROUP_SIZE[precision]
        self.K, self.N, self.rank, self.precision = K, N, rank, precision
        self.packed_w = t((N, K // 2), U8)
        self.wscales = t((N, K // G), BF if precision == "int4" else U8)
        self.smooth = t((K,))
        self.lora_down = t((rank, K)) if rank else None
        self.lora_up = t((N, rank)) if rank else None
        self.bias = t((N,))
        self.wtscale = 1.0

    def workspace_bytes(self, M):
        return 1 << 20


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def svdq_args(K=256, N=192, rank=16, precision="int4", **over):
    G = bq.GROUP_SIZE[precision]
    d = dict(packed_w=t((N, K // 2), U8), wscales=t((N, K // G), BF if precision == "int4" else U8),
             smooth=t((K,)), lora_down=t((rank, K)), lora_up=t((N, rank)), bias=t((N,)), precision=precision)
    d.update(over)
    return d


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_svdq_layer_constructor(precision):
    G = bq.GROUP_SIZE[precision]
    sdt = BF if precision == "int4" else U8
    # a well-formed layer on the CPU gets as far as the device check
    raises("must be a CUDA tensor", bq.SVDQLinear, **svdq_args(precision=precision))
    bad = {
        "packed_w": t((192, 128, 1), U8),
        "wscales": t((192, 256 // G + 1), sdt),
        "smooth": t((255,)),
        "lora_down": t((16, 128)),
        "lora_up": t((191, 16)),
        "bias": t((193,)),
    }
    for name, v in bad.items():
        raises(f"{name} must have shape", bq.SVDQLinear, **svdq_args(precision=precision, **{name: v}))
    raises("wscales must have dtype", bq.SVDQLinear,
           **svdq_args(precision=precision, wscales=t((192, 256 // G), F32)))
    raises("smooth must have dtype", bq.SVDQLinear, **svdq_args(precision=precision, smooth=t((256,), F32)))
    raises("packed_w must be contiguous", bq.SVDQLinear,
           **svdq_args(precision=precision, packed_w=t((128, 192), U8).t()))
    raises("both be given or both be None", bq.SVDQLinear, **svdq_args(precision=precision, lora_up=None))
    raises("precision must be one of", bq.SVDQLinear, **dict(svdq_args(), precision="int8"))


def test_svdq_linear_call():
    L = FakeLayer()
    raises("x must have shape", bq.svdq_w4a4_linear, t((8, 128)), L)
    raises("x must have shape", bq.svdq_w4a4_linear, t((8, 256, 1)), L)
    raises("x must have dtype", bq.svdq_w4a4_linear, t((8, 256), F32), L)
    raises("out must have shape", bq.svdq_w4a4_linear, t((8, 256)), L, out=t((8, 191)))
    raises("out must have dtype", bq.svdq_w4a4_linear, t((8, 256)), L, out=t((8, 192), F32))
    raises("out must be contiguous", bq.svdq_w4a4_linear, t((8, 256)), L, out=t((192, 8)).t())
    raises("workspace must have dtype", bq.svdq_w4a4_linear, t((8, 256)), L, out=t((8, 192)),
           workspace=t((64,), F32))
    raises("workspace must have shape", bq.svdq_w4a4_linear, t((8, 256)), L, out=t((8, 192)),
           workspace=t((8, 8), U8))
    raises("must be a CUDA tensor", bq.svdq_w4a4_linear, t((8, 256)), L, out=t((8, 192)),
           workspace=t((64,), U8))
    # the two-phase entry points
    raises("x must have shape", bq.svdq_w4a4_quantize, t((8, 128)), L, t((64,), U8))
    raises("workspace must have dtype", bq.svdq_w4a4_quantize, t((8, 256)), L, t((64,), F32))
    raises("out must have shape", bq.svdq_w4a4_gemm, t((64,), U8), 8, L, out=t((8, 64)))


def test_mlp_and_qkv_calls():
    up, down = FakeLayer(K=256, N=384), FakeLayer(K=384, N=256, precision="nvfp4")
    raises("must equal the down layer's K", bq.svdq_w4a4_mlp_gelu, t((8, 256)), up, FakeLayer(K=256, N=256))
    raises("x must have shape", bq.svdq_w4a4_mlp_gelu, t((8, 384)), up, down)
    raises("out must have shape", bq.svdq_w4a4_mlp_gelu, t((8, 256)), up, down, out=t((8, 384)))
    qkv = FakeLayer(K=256, N=384)
    ok = dict(q_norm=t((128,)), k_norm=t((128,)), rope_cos=t((8, 64), F32), rope_sin=t((8, 64), F32))

    def call(x=None, **kw):
        a = dict(ok)
        a.update(kw)
        return bq.svdq_w4a4_qkv_rmsnorm_rope(t((8, 256)) if x is None else x, qkv, 1, a["q_norm"], a["k_norm"],
                                             a["rope_cos"], a["rope_sin"], out=a.get("out"))
    raises("x must have shape", call, x=t((8, 255)))
    raises("k_norm must have shape", call, k_norm=t((64,)))
    raises("rope_cos must have shape", call, rope_cos=t((7, 64), F32))
    raises("rope_sin must have shape", call, rope_sin=t((8, 32), F32))
    raises("rope_cos must have dtype", call, rope_cos=t((8, 64)))
    raises("out must have shape", call, out=t((8, 383)))


def test_awq_layer_and_call():
    ok = dict(packed_w=t((128, 128), U8), wscales=t((128, 4)), wzeros=t((128, 4)), bias=t((128,)))
    raises("must be a CUDA tensor", bq.AWQLinear, **ok)
    for name, v in {"wscales": t((128, 3)), "wzeros": t((127, 4)), "bias": t((64,))}.items():
        d = dict(ok)
        d[name] = v
        raises(f"{name} must have shape", bq.AWQLinear, **d)

    class A:
        K, N = 256, 128
    raises("x must have shape", bq.awq_w4a16_linear, t((2, 128)), A())
    raises("out must have shape", bq.awq_w4a16_linear, t((2, 256)), A(), out=t((1, 128)))


def test_parity_exports():
    raises("smooth must have shape", bq.svdq_w4a4_quantize_act, t((8, 256)), t((128,)), None, "int4")
    raises("lora_down must have shape", bq.svdq_w4a4_quantize_act, t((8, 256)), t((256,)), t((16, 128)), "int4")
    raises("codes must have shape", bq.svdq_w4a4_quantize_act, t((8, 256)), t((256,)), None, "int4",
           out=(t((8, 64), U8), t((8, 4)), None))
    raises("scales must have dtype", bq.svdq_w4a4_quantize_act, t((8, 256)), t((256,)), None, "nvfp4",
           out=(t((8, 128), U8), t((8, 16)), None))
    raises("smooth must have shape", bq.svdq_w4a4_quantize_operand, t((8, 256)), t((255,)), None, "nvfp4")
    raises("precision must be one of", bq.svdq_w4a4_quantize_operand, t((8, 256)), t((256,)), None, "fp8")
    raises("w_codes must have shape", bq.svdq_w4a4_gemm_partials, t((8, 128), U8), t((64, 64), U8), "int4")
    raises("act_codes must have dtype", bq.svdq_w4a4_gemm_partials, t((8, 128)), t((64, 128), U8), "int4")


def test_weight_prep_calls():
    raises("x_calib must have shape", bq.smooth_factors, t((16, 128)), t((64, 256), F32))
    raises("w must have dtype", bq.smooth_factors, t((16, 256)), t((64, 256)))
    raises("resid must have shape", bq.pack_weight, t((64,), F32), "int4")
    raises("precision must be one of", bq.pack_weight, t((64, 256), F32), "int8")
