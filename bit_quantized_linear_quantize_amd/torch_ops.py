"""The two linears as ``torch.library`` custom ops, so that models calling
them trace into ``torch.compile(fullgraph=True)`` graphs without breaks.

Each op allocates its output (and, for svdq_w4a4, its workspace) with the
caching allocator and calls the same C ABI as the rest of the binding, on the
current stream; the fake implementations give the output shape and dtype for
tracing.  Nothing here computes: the arithmetic is in the HIP kernels.

    torch.ops.svdq.w4a4_linear(x, packed_w, wscales, wtscale, smooth,
                               lora_down, lora_up, bias, precision) -> Tensor
    torch.ops.svdq.awq_w4a16_linear(x, packed_w, wscales, wzeros, bias) -> Tensor
    torch.ops.svdq.w4a4_mlp_gelu(x, <up layer tensors>, <down layer tensors>) -> Tensor
    torch.ops.svdq.w4a4_qkv_rmsnorm_rope(x, <layer tensors>, heads, q_norm, k_norm,
                                         rope_cos, rope_sin, eps) -> Tensor

``svdq_linear(x, layer)``, ``awq_linear(x, layer)``, ``mlp_gelu(x, up, down)``
and ``qkv_rmsnorm_rope(x, layer, heads, ...)`` call them with the tensors of
``SVDQLinear`` / ``AWQLinear`` objects.
"""

from typing import Optional

import torch

from . import (AWQLinear, SVDQLinear, awq_w4a16_linear, svdq_w4a4_linear, svdq_w4a4_mlp_gelu,
               svdq_w4a4_qkv_rmsnorm_rope)


@torch.library.custom_op("svdq::w4a4_linear", mutates_args=())
def w4a4_linear(x: torch.Tensor, packed_w: torch.Tensor, wscales: torch.Tensor, wtscale: float,
                smooth: torch.Tensor, lora_down: Optional[torch.Tensor], lora_up: Optional[torch.Tensor],
                bias: Optional[torch.Tensor], precision: str) -> torch.Tensor:
    layer = SVDQLinear(packed_w, wscales, smooth, lora_down, lora_up, bias, precision, wtscale)
    return svdq_w4a4_linear(x, layer)


@w4a4_linear.register_fake
def _w4a4_linear_fake(x, packed_w, wscales, wtscale, smooth, lora_down, lora_up, bias, precision):
    return x.new_empty((x.shape[0], packed_w.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("svdq::awq_w4a16_linear", mutates_args=())
def awq_linear_op(x: torch.Tensor, packed_w: torch.Tensor, wscales: torch.Tensor, wzeros: torch.Tensor,
                  bias: Optional[torch.Tensor]) -> torch.Tensor:
    return awq_w4a16_linear(x, AWQLinear(packed_w, wscales, wzeros, bias))


@awq_linear_op.register_fake
def _awq_linear_fake(x, packed_w, wscales, wzeros, bias):
    return x.new_empty((x.shape[0], packed_w.shape[0]), dtype=torch.bfloat16)


def svdq_linear(x, layer):
    """svdq_w4a4 linear of an ``SVDQLinear`` through the custom op."""
    return torch.ops.svdq.w4a4_linear(x, layer.packed_w, layer.wscales, layer.wtscale, layer.smooth,
                                      layer.lora_down, layer.lora_up, layer.bias, layer.precision)


def awq_linear(x, layer):
    """awq_w4a16 linear of an ``AWQLinear`` through the custom op."""
    return torch.ops.svdq.awq_w4a16_linear(x, layer.packed_w, layer.wscales, layer.wzeros, layer.bias)


@torch.library.custom_op("svdq::w4a4_mlp_gelu", mutates_args=())
def w4a4_mlp_gelu(x: torch.Tensor, up_packed_w: torch.Tensor, up_wscales: torch.Tensor, up_wtscale: float,
                  up_smooth: torch.Tensor, up_lora_down: Optional[torch.Tensor], up_lora_up: Optional[torch.Tensor],
                  up_bias: Optional[torch.Tensor], up_precision: str, dn_packed_w: torch.Tensor,
                  dn_wscales: torch.Tensor, dn_wtscale: float, dn_smooth: torch.Tensor,
                  dn_lora_down: Optional[torch.Tensor], dn_lora_up: Optional[torch.Tensor],
                  dn_bias: Optional[torch.Tensor]) -> torch.Tensor:
    up = SVDQLinear(up_packed_w, up_wscales, up_smooth, up_lora_down, up_lora_up, up_bias, up_precision, up_wtscale)
    down = SVDQLinear(dn_packed_w, dn_wscales, dn_smooth, dn_lora_down, dn_lora_up, dn_bias, "nvfp4", dn_wtscale)
    return svdq_w4a4_mlp_gelu(x, up, down)


@w4a4_mlp_gelu.register_fake
def _w4a4_mlp_gelu_fake(x, up_packed_w, up_wscales, up_wtscale, up_smooth, up_lora_down, up_lora_up, up_bias,
                        up_precision, dn_packed_w, *rest):
    return x.new_empty((x.shape[0], dn_packed_w.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("svdq::w4a4_qkv_rmsnorm_rope", mutates_args=())
def w4a4_qkv_rmsnorm_rope(x: torch.Tensor, packed_w: torch.Tensor, wscales: torch.Tensor, wtscale: float,
                          smooth: torch.Tensor, lora_down: Optional[torch.Tensor], lora_up: Optional[torch.Tensor],
                          bias: Optional[torch.Tensor], precision: str, heads: int, q_norm: torch.Tensor,
                          k_norm: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                          eps: float) -> torch.Tensor:
    layer = SVDQLinear(packed_w, wscales, smooth, lora_down, lora_up, bias, precision, wtscale)
    return svdq_w4a4_qkv_rmsnorm_rope(x, layer, heads, q_norm, k_norm, rope_cos, rope_sin, eps)


@w4a4_qkv_rmsnorm_rope.register_fake
def _w4a4_qkv_fake(x, packed_w, *rest):
    return x.new_empty((x.shape[0], packed_w.shape[0]), dtype=torch.bfloat16)


def _layer_args(layer):
    return (layer.packed_w, layer.wscales, layer.wtscale, layer.smooth, layer.lora_down, layer.lora_up, layer.bias)


def mlp_gelu(x, up, down):
    """The fused GELU MLP of two ``SVDQLinear`` (down: nvfp4) through the custom op."""
    return torch.ops.svdq.w4a4_mlp_gelu(x, *_layer_args(up), up.precision, *_layer_args(down))


def qkv_rmsnorm_rope(x, layer, heads, q_norm, k_norm, rope_cos, rope_sin, eps=1e-6):
    """The fused QKV projection with RMSNorm and RoPE through the custom op."""
    return torch.ops.svdq.w4a4_qkv_rmsnorm_rope(x, *_layer_args(layer), layer.precision, heads, q_norm, k_norm,
                                                rope_cos, rope_sin, eps)
