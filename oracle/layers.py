"""Weight preparation and reference quantized linears (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Conventions (readings; the pages define no layouts):

* Linear layers follow the ``nn.Linear`` convention the pages' targets use
  ("NunchakuLiteQuantizationConfig" section: every target is a linear layer):
  X [M, K], W [N, K], Y = X W^T + b, Y [M, N].
* The low-rank branch is two bfloat16 linears in the same convention:
  ``lora_down`` [r, K] (K -> r) and ``lora_up`` [N, r] (r -> N), so the branch
  adds (X_hat lora_down^T) lora_up^T.  Rank 32 is the example's ``rank``.
* bfloat16 tensors are uint16 bit patterns; E4M3 scales are uint8 codes;
  packed codes are uint8 [rows, K/2] with the low nibble = even column.

SVDQ (the "Supported quantization types" table: 4-bit weights and
activations "with SVDQ low-rank correction"; the news article's account:
outliers move into a 16-bit low-rank branch) -- readings, in order:

1. smoothing factor per input channel: lambda_k = sqrt(amax_x[k] / amax_w[k])
   (1 where that is zero or not finite), stored as bf16 ``smooth``;
2. the layer divides activations by ``smooth`` and multiplies the weight by it,
   W_hat[n, k] = W[n, k] * smooth_k, so X_hat W_hat^T = X W^T;
3. W_hat = U Sigma V^T (fp64 SVD); lora_down = Sigma_r V_r^T, lora_up = U_r,
   both rounded to bf16;
4. residual R = W_hat - lora_up lora_down (fp64, from the bf16 factors, the
   rank terms added in order), cast to fp32 and quantized per row with the
   activation quantizer of the precision (nvfp4 adds one fp32 tensor scale);
5. forward: X_hat = fl32(x * fl32(1/smooth)); quantize X_hat per token;
   Y = sum_g P_g * s_a * s_w * c + (X_hat lora_down^T) lora_up^T + bias,
   accumulated in fp64, with P_g the integer dot product of the codes in group
   g (nvfp4 uses doubled E2M1 codes, c = t_w / 4; int4 has c = 1).

AWQ (table row ``awq_w4a16``, int4 weight-only, group 64): y = x W_deq^T + b,
W_deq = (q - z) * s, fp64 accumulation.
"""

import numpy as np

from .formats import (F32, bf16_bits, bf16_bits_f64, bf16_to_f32, e4m3_decode,
                      e2m1_decode, e4m3_encode, pack_nibbles, nibble_to_int4)
from .quant import (quantize_int4, quantize_nvfp4_act, quantize_nvfp4_weight,
                    quantize_awq)

GROUP = {"int4": 64, "nvfp4": 16}


# ----------------------------------------------------------------------------
# weight preparation
# ----------------------------------------------------------------------------
def smooth_factors(x_bits, w):
    """Per-channel smoothing factors sqrt(amax_x / amax_w) as bf16 bits [K]."""
    x = np.abs(bf16_to_f32(x_bits).astype(np.float64))
    w = np.abs(np.asarray(w, dtype=np.float64))
    amax_x = x.max(axis=0)
    amax_w = w.max(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lam = np.sqrt(amax_x / amax_w)
    lam = np.where(np.isfinite(lam) & (lam > 0), lam, 1.0)
    return bf16_bits_f64(lam)


def prepare_svdq_layer(w, smooth_bits, rank, precision, bias_bits=None):
    """Offline SVDQ preparation of one linear.

    ``w``: float64 [N, K] original weight; ``smooth_bits``: bf16 bits [K].
    Returns a dict with the library's inputs (packed_w, wscales, wtscale,
    smooth, lora_down, lora_up, bias) plus the integer codes and the singular
    values for the oracle's own checks.
    """
    if precision not in GROUP:
        raise ValueError(precision)
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    smooth = bf16_to_f32(smooth_bits).astype(np.float64)
    w_hat = w * smooth[None, :]
    u, sig, vt = np.linalg.svd(w_hat, full_matrices=False)
    down = sig[:rank, None] * vt[:rank, :]          # [r, K]
    up = u[:, :rank]                                # [N, r]
    down_bits = bf16_bits_f64(down).reshape(rank, K)
    up_bits = bf16_bits_f64(up).reshape(N, rank)
    out = prepare_svdq_layer_from_factors(w, smooth_bits, down_bits, up_bits, precision, bias_bits)
    out["sigma"] = sig
    return out


def low_rank_residual(w, smooth_bits, down_bits, up_bits):
    """R = W_hat - lora_up lora_down in fp64 from the bf16 factors, with
    W_hat[n, k] = w[n, k] * smooth[k].  The r terms of each entry are added in
    order j = 0 .. r-1, each product rounded to fp64 on its own (reading: the
    pages give no arithmetic; a fixed order makes the residual reproducible
    bit for bit by any implementation, whatever its matrix-product library).
    Returns (W_hat, R) as float64 [N, K]."""
    w = np.asarray(w, dtype=np.float64)
    smooth = bf16_to_f32(smooth_bits).astype(np.float64)
    w_hat = w * smooth[None, :]
    up = bf16_to_f32(up_bits).astype(np.float64)
    down = bf16_to_f32(down_bits).astype(np.float64)
    low = np.zeros_like(w_hat)
    for j in range(up.shape[1]):
        low = low + up[:, j:j + 1] * down[j:j + 1, :]
    return w_hat, w_hat - low


def prepare_svdq_layer_from_factors(w, smooth_bits, down_bits, up_bits, precision, bias_bits=None):
    """The rest of the preparation given the bf16 low-rank factors
    (lora_down [r, K], lora_up [N, r]): the residual (low_rank_residual), cast
    to fp32, quantized per row and packed.  Same dict as prepare_svdq_layer,
    without the singular values."""
    if precision not in GROUP:
        raise ValueError(precision)
    G = GROUP[precision]
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    down_bits = np.asarray(down_bits, np.uint16).reshape(-1, K)
    up_bits = np.asarray(up_bits, np.uint16).reshape(N, -1)
    rank = down_bits.shape[0]
    w_hat, resid = low_rank_residual(w, smooth_bits, down_bits, up_bits)
    r32 = resid.astype(F32)
    out = dict(precision=precision, group_size=G, rank=rank, N=N, K=K,
               smooth=np.asarray(smooth_bits, np.uint16), lora_down=down_bits,
               lora_up=up_bits, w_hat=w_hat, resid=resid,
               bias=None if bias_bits is None else np.asarray(bias_bits, np.uint16))
    if precision == "int4":
        nib, s, q = quantize_int4(r32, G)
        out.update(packed_w=pack_nibbles(nib), wscales=bf16_bits(s), wtscale=1.0,
                   w_codes=nib, w_int=q)
    else:
        codes, s8, t = quantize_nvfp4_weight(r32, G)
        out.update(packed_w=pack_nibbles(codes), wscales=s8, wtscale=t,
                   w_codes=codes)
    return out


def prepare_awq_layer(w, bias_bits=None, G=64):
    """AWQ W4A16 preparation: packed uint4 codes, bf16 scales and zero-points."""
    w32 = np.asarray(w, dtype=np.float64).astype(F32)
    q, s, z = quantize_awq(w32, G)
    return dict(packed_w=pack_nibbles(q), wscales=bf16_bits(s), wzeros=bf16_bits(z),
                q=q, group_size=G, N=w32.shape[0], K=w32.shape[1],
                bias=None if bias_bits is None else np.asarray(bias_bits, np.uint16))


# ----------------------------------------------------------------------------
# activation side
# ----------------------------------------------------------------------------
def smoothed_activations(x_bits, smooth_bits):
    """X_hat = fl32(x * fl32(1 / smooth)) as float32 [M, K]."""
    x = bf16_to_f32(x_bits)
    mu = (F32(1.0) / bf16_to_f32(smooth_bits)).astype(F32)
    return (x * mu[None, :]).astype(F32)


def svdq_quantize_act(x_bits, smooth_bits, lora_down_bits, precision):
    """Activation quantizer + low-rank down projection.

    Returns dict(codes [M, K] nibbles, packed [M, K/2], scales (bf16 bits
    [M, K/64] for int4, E4M3 codes [M, K/16] for nvfp4), lora_act float64
    [M, r], xhat float32 [M, K]).
    """
    G = GROUP[precision]
    xhat = smoothed_activations(x_bits, smooth_bits)
    if precision == "int4":
        nib, s, _ = quantize_int4(xhat, G)
        scales = bf16_bits(s)
    else:
        nib, scales = quantize_nvfp4_act(xhat, G)
    down = bf16_to_f32(lora_down_bits).astype(np.float64)
    lora_act = xhat.astype(np.float64) @ down.T if down.shape[0] else np.zeros((xhat.shape[0], 0))
    return dict(codes=nib, packed=pack_nibbles(nib), scales=scales, lora_act=lora_act, xhat=xhat)


def product_operand_ref(codes, scales, precision):
    """The activations as the product kernel receives them.

    Reading (the pages fix no operand format; this is the library's own
    encoding of the activation codes and group scales, defined here value by
    value):
      nvfp4: the dequantized value e2m1 * dec(s8), always an exact binary16
             (|v| <= 2688, nonzero |v| >= 2^-10); no separate scales (None).
      int4:  each code q (|q| <= 7, sign-magnitude) as an OCP fp8 E4M3 byte --
             every such integer is an E4M3 value, and the code 0x8 ("-0")
             keeps its sign (0x80) -- and the group scales s as float64
             [R, K/64] (the bf16 values).  The product kernel forms each
             group's exact integer sum P and adds P * (s_x * s_w).

    codes [R, K] nibbles; scales as returned by the quantizers ([R, K/G]).
    Returns (nvfp4: values float64 [R, K], None; int4: E4M3 bytes uint8
    [R, K], scales float64 [R, K/64]).
    """
    G = GROUP[precision]
    if precision == "nvfp4":
        q = _code_values(codes, precision)
        s = _scale_values(scales, precision)
        R, K = q.shape
        return (q.reshape(R, K // G, G) * s[..., None]).reshape(R, K), None
    n = np.asarray(codes, dtype=np.uint8)
    mag = (n & 7).astype(np.float64)
    signed = np.where((n & 8) != 0, -mag, mag)  # -0.0 for the code 0x8
    return e4m3_encode(signed), _scale_values(scales, precision)


def _code_values(codes, precision):
    """Nibble codes -> exact values: int4 integers, or E2M1 values."""
    if precision == "int4":
        return nibble_to_int4(codes).astype(np.float64)
    return e2m1_decode(codes).astype(np.float64)


def _scale_values(scales, precision):
    if precision == "int4":
        return bf16_to_f32(scales).astype(np.float64)
    return e4m3_decode(scales).astype(np.float64)


def dequant(codes, scales, precision):
    """Codes [R, K] and group scales [R, K/G] -> exact float64 values."""
    G = GROUP[precision]
    v = _code_values(codes, precision)
    s = _scale_values(scales, precision)
    R, K = v.shape
    return (v.reshape(R, K // G, G) * s[..., None]).reshape(R, K)


# ----------------------------------------------------------------------------
# reference forward passes
# ----------------------------------------------------------------------------
def svdq_linear_ref(x_bits, layer, act=None):
    """Reference SVDQ W4A4 forward in fp64: returns Y [M, N] float64."""
    p = layer["precision"]
    if act is None:
        act = svdq_quantize_act(x_bits, layer["smooth"], layer["lora_down"], p)
    a = dequant(act["codes"], act["scales"], p)
    w = dequant(layer["w_codes"], layer["wscales"], p)
    y = (a @ w.T) * float(layer["wtscale"])
    if layer["rank"]:
        y = y + act["lora_act"] @ bf16_to_f32(layer["lora_up"]).astype(np.float64).T
    if layer.get("bias") is not None:
        y = y + bf16_to_f32(layer["bias"]).astype(np.float64)[None, :]
    return y


def svdq_partials_ref(act_codes, w_codes, precision):
    """Exact per-group integer dot products P[m, n, g] (int64).

    int4 uses the signed codes; nvfp4 uses doubled E2M1 codes (integers in
    {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}).
    """
    G = GROUP[precision]
    if precision == "int4":
        a = nibble_to_int4(act_codes)
        w = nibble_to_int4(w_codes)
    else:
        a = np.rint(2 * e2m1_decode(act_codes)).astype(np.int64)
        w = np.rint(2 * e2m1_decode(w_codes)).astype(np.int64)
    M, K = a.shape
    N = w.shape[0]
    return np.einsum("mgk,ngk->mng", a.reshape(M, K // G, G), w.reshape(N, K // G, G))


def gelu_f64(y):
    """GELU with the exact erf, y/2 (1 + erf(y / sqrt 2)), in fp64 (the
    activation between the two linears of the DiT MLP), written as
    y/2 erfc(-y / sqrt 2): the same function, without the cancellation of
    1 + erf for negative y (scipy's erfc is the library routine)."""
    from scipy.special import erfc
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * erfc(-y / np.sqrt(2.0))


def gelu_bf16(y_bits):
    """A bf16 GELU of bf16 values: gelu_f64 of the values, rounded once to
    bf16 (RNE).  Takes and returns bf16 bit patterns."""
    return bf16_bits_f64(gelu_f64(bf16_to_f32(y_bits).astype(np.float64)))


def mlp_gelu_ref(h_bits, down):
    """Reference of the GELU MLP's second half, given the up projection's bf16
    output h: the down linear (svdq_linear_ref) of gelu_bf16(h), in fp64.
    (The fused MLP computes the same hidden values; h itself is the up
    linear, checked on its own.)"""
    return svdq_linear_ref(gelu_bf16(h_bits), down)


# ----------------------------------------------------------------------------
# fused QKV projection with RMSNorm and RoPE ("Fused kernels" section of the
# Nunchaku Lite docs: the original engine merges the Q, K and V projections
# with RMSNorm and RoPE).  Readings: the layout is one [M, 3 H D] output
# q | k | v, heads of D consecutive columns; q and k get a per-head RMSNorm
# with their own learned weights [D], then the rotary embedding on interleaved
# pairs (2i, 2i+1) with per-token angle tables; v is the projection itself.
# The value chain is that of separate bf16 ops: h = bf16(linear), n =
# bf16(RMSNorm(h)), out = bf16(RoPE(n)).
# ----------------------------------------------------------------------------
def rmsnorm_bf16(h_bits, w_bits, eps):
    """RMSNorm over the last axis of bf16 values: h / sqrt(mean(h^2) + eps) * w,
    in fp64, rounded once to bf16.  Takes and returns bf16 bit patterns."""
    h = bf16_to_f32(h_bits).astype(np.float64)
    w = bf16_to_f32(w_bits).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + float(eps))
    return bf16_bits_f64(h * r * w)


def rope_f64(n, cos, sin):
    """Rotary embedding on interleaved pairs of the last axis, in fp64:
    (a, b) at columns (2i, 2i+1) -> (a cos_i - b sin_i, a sin_i + b cos_i).
    n [..., D] float; cos, sin [..., D/2] broadcast against n's leading axes."""
    n = np.asarray(n, dtype=np.float64)
    a, b = n[..., 0::2], n[..., 1::2]
    c, s = np.asarray(cos, np.float64), np.asarray(sin, np.float64)
    out = np.empty_like(n)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qkv_norm_rope_ref(x_bits, layer, heads, q_norm_bits, k_norm_bits, eps, cos, sin):
    """Reference of the fused QKV projection + RMSNorm + RoPE, fp64.

    x [M, K] bf16 bits; ``layer`` a prepared svdq layer with N = 3 heads D;
    q_norm / k_norm bf16 bits [D]; cos, sin float32 [M, D/2] (per token).
    Returns [M, N] float64: q and k columns are RoPE(RMSNorm(bf16(h))) before
    the final bf16 rounding, v columns are the linear's own fp64 output."""
    h64 = svdq_linear_ref(x_bits, layer)
    M, N = h64.shape
    D = N // (3 * heads)
    h = bf16_bits_f64(h64)
    out = h64.copy()
    for part, wb in ((0, q_norm_bits), (1, k_norm_bits)):
        cols = slice(part * heads * D, (part + 1) * heads * D)
        hp = h[:, cols].reshape(M, heads, D)
        n = bf16_to_f32(rmsnorm_bf16(hp, wb, eps)).astype(np.float64)
        out[:, cols] = rope_f64(n, np.asarray(cos)[:, None, :], np.asarray(sin)[:, None, :]).reshape(M, heads * D)
    return out


def awq_dequant(layer):
    G = layer["group_size"]
    q = layer["q"].astype(np.float64)
    N, K = q.shape
    s = bf16_to_f32(layer["wscales"]).astype(np.float64)
    z = bf16_to_f32(layer["wzeros"]).astype(np.float64)
    return ((q.reshape(N, K // G, G) - z[..., None]) * s[..., None]).reshape(N, K)


def awq_linear_ref(x_bits, layer):
    """Reference AWQ W4A16 forward in fp64: y = x W_deq^T + bias."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    y = x @ awq_dequant(layer).T
    if layer.get("bias") is not None:
        y = y + bf16_to_f32(layer["bias"]).astype(np.float64)[None, :]
    return y


# ----------------------------------------------------------------------------
# error metrics used by the parity tests
# ----------------------------------------------------------------------------
def bf16_half_ulp(y):
    """Half the bfloat16 spacing at |y| (float64): the largest error of
    rounding y to bfloat16.  bfloat16 has 8 significant bits, so in the
    binade [2^e, 2^(e+1)) its spacing is 2^(e-7); below 2^-126 the spacing of
    its subnormals, 2^-133.  The binade comes from ``np.frexp`` (exact: a
    value just below a power of two stays in the lower binade)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(a)  # a = m 2^e, 0.5 <= m < 1: a lies in [2^(e-1), 2^e)
    e = np.maximum(np.where(a > 0, e - 1, -126), -126)
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def output_errors(y_gpu, y_ref):
    """(max|err| / RMS(y_ref), max of (|err| - half-ulp) / RMS, mean relative error)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2)) if y_ref.size else 0.0
    excess = np.max(err - bf16_half_ulp(y_ref)) if y_ref.size else 0.0
    mre = err.sum() / max(np.abs(y_ref).sum(), 1e-300)
    return (err.max() / rms if rms else err.max()), (excess / rms if rms else excess), mre
