"""The two linears as ``torch.library`` custom ops, so that models calling
them trace into ``torch.compile(fullgraph=True)`` graphs without breaks.

Each op allocates its output (and, for svdq_w4a4, its workspace) with the
caching allocator and calls the same C ABI as the rest of the binding, on the
current stream; the fake implementations give the output shape and dtype for
tracing.  Nothing here computes: the arithmetic is in the HIP kernels.

    torch.ops.svdq.w4a4_linear(x, packed_w, wscales, wtscale, smooth,
                               lora_down, lora_up, bias, precision) -> Tensor
    torch.ops.svdq.awq_w4a16_linear(x, packed_w, wscales, wzeros, bias) -> Tensor

``svdq_linear(x, layer)`` and ``awq_linear(x, layer)`` call them with the
tensors of an ``SVDQLinear`` / ``AWQLinear``.
"""

from typing import Optional

import torch

from . import AWQLinear, SVDQLinear, awq_w4a16_linear, svdq_w4a4_linear


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
