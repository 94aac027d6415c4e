"""Thin Python binding of the gfx950 SVDQ W4A4 / AWQ W4A16 library.

Argument marshalling only: every step of the quantized linears runs in the HIP
kernels of ``lib/libsvdq_w4a4.so`` (built by ``build.py``) behind the C ABI of
``include/svdq_w4a4.h``.  PyTorch provides device memory and the current HIP
stream.  There is no fallback: if the library is missing or the call fails,
an exception is raised.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libsvdq_w4a4.so")

SVDQ_INT4 = 0
SVDQ_NVFP4 = 1
PRECISIONS = {"int4": SVDQ_INT4, "nvfp4": SVDQ_NVFP4}
GROUP_SIZE = {"int4": 64, "nvfp4": 16}
STATUS = {0: "SVDQ_OK", -1: "SVDQ_EINVAL", -2: "SVDQ_EUNSUPPORTED", -3: "SVDQ_EARCH",
          -4: "SVDQ_EWORKSPACE", -5: "SVDQ_EDEVICE"}

# entry points declared in include/svdq_w4a4.h
EXPORTS = ("svdq_w4a4_workspace_bytes", "svdq_w4a4_linear", "svdq_w4a4_linear_noalloc", "svdq_w4a4_quantize",
           "svdq_w4a4_gemm",
           "awq_w4a16_linear", "svdq_w4a4_mlp_workspace_bytes", "svdq_w4a4_mlp_gelu",
           "svdq_w4a4_quantize_act", "svdq_w4a4_quantize_operand", "svdq_w4a4_gemm_partials",
           "svdq_w4a4_check",
           "awq_w4a16_check", "svdq_w4a4_mlp_gelu_check", "svdq_w4a4_qkv_rmsnorm_rope",
           "svdq_w4a4_qkv_rmsnorm_rope_check", "svdq_w4a4_prep_workspace_bytes", "svdq_w4a4_smooth_factors",
           "svdq_w4a4_pack_weight", "svdq_w4a4_prepare_workspace_bytes", "svdq_w4a4_prepare_weight",
           "svdq_w4a4_gelu_table", "svdq_last_error")


class LayerStruct(ctypes.Structure):
    """svdq_w4a4_layer of include/svdq_w4a4.h."""
    _fields_ = [("packed_w", ctypes.c_void_p), ("wscales", ctypes.c_void_p), ("wtscale", ctypes.c_float),
                ("smooth", ctypes.c_void_p), ("lora_down", ctypes.c_void_p), ("lora_up", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("precision", ctypes.c_int), ("group_size", ctypes.c_int), ("rank", ctypes.c_int)]


class SvdqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
P = ctypes.c_void_p
I64 = ctypes.c_int64
I = ctypes.c_int


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.svdq_w4a4_workspace_bytes.argtypes = [I64, I64, I64, I, I, I]
        L.svdq_w4a4_workspace_bytes.restype = ctypes.c_size_t
        L.svdq_w4a4_linear.argtypes = [P, I64, I64, I64, P, P, ctypes.c_float, P, P, P, P, I, I, I,
                                       P, P, ctypes.c_size_t, P]
        L.svdq_w4a4_linear.restype = I
        L.svdq_w4a4_linear_noalloc.argtypes = [P, I64, I64, I64, P, P, ctypes.c_float, P, P, P, P, I, I, I, P, P]
        L.svdq_w4a4_linear_noalloc.restype = I
        L.svdq_w4a4_quantize.argtypes = [P, I64, I64, P, P, I, I, I, P, ctypes.c_size_t, P]
        L.svdq_w4a4_quantize.restype = I
        L.svdq_w4a4_gemm.argtypes = [P, ctypes.c_size_t, I64, I64, I64, P, P, ctypes.c_float, P, P, I, I, I,
                                     P, P]
        L.svdq_w4a4_gemm.restype = I
        L.awq_w4a16_linear.argtypes = [P, I64, I64, I64, P, P, P, P, I, P, P]
        L.awq_w4a16_linear.restype = I
        L.svdq_w4a4_quantize_act.argtypes = [P, I64, I64, P, P, I, I, I, P, P, P, P]
        L.svdq_w4a4_quantize_act.restype = I
        L.svdq_w4a4_quantize_operand.argtypes = [P, I64, I64, P, P, I, I, I, P, P, P, P]
        L.svdq_w4a4_quantize_operand.restype = I
        L.svdq_w4a4_gemm_partials.argtypes = [P, P, I64, I64, I64, I, I, P, P]
        L.svdq_w4a4_gemm_partials.restype = I
        L.svdq_w4a4_check.argtypes = [P, I64, I64, I64, P, P, ctypes.c_float, P, P, P, P, I, I, I,
                                      P, P, ctypes.c_size_t, ctypes.c_char_p]
        L.svdq_w4a4_check.restype = I
        L.awq_w4a16_check.argtypes = [P, I64, I64, I64, P, P, P, P, I, P, ctypes.c_char_p]
        L.awq_w4a16_check.restype = I
        LP = ctypes.POINTER(LayerStruct)
        L.svdq_w4a4_mlp_workspace_bytes.argtypes = [I64, LP, LP]
        L.svdq_w4a4_mlp_workspace_bytes.restype = ctypes.c_size_t
        L.svdq_w4a4_mlp_gelu.argtypes = [P, I64, LP, LP, P, P, ctypes.c_size_t, P]
        L.svdq_w4a4_mlp_gelu.restype = I
        L.svdq_w4a4_mlp_gelu_check.argtypes = [P, I64, LP, LP, P, P, ctypes.c_size_t, ctypes.c_char_p]
        L.svdq_w4a4_mlp_gelu_check.restype = I
        F = ctypes.c_float
        L.svdq_w4a4_qkv_rmsnorm_rope.argtypes = [P, I64, LP, I, I, P, P, F, P, P, P, P, ctypes.c_size_t, P]
        L.svdq_w4a4_qkv_rmsnorm_rope.restype = I
        L.svdq_w4a4_qkv_rmsnorm_rope_check.argtypes = [P, I64, LP, I, I, P, P, F, P, P, P, P, ctypes.c_size_t,
                                                       ctypes.c_char_p]
        L.svdq_w4a4_qkv_rmsnorm_rope_check.restype = I
        L.svdq_w4a4_prep_workspace_bytes.argtypes = [I64]
        L.svdq_w4a4_prep_workspace_bytes.restype = ctypes.c_size_t
        L.svdq_w4a4_smooth_factors.argtypes = [P, I64, P, I64, I64, P, P, ctypes.c_size_t, P]
        L.svdq_w4a4_smooth_factors.restype = I
        L.svdq_w4a4_pack_weight.argtypes = [P, I64, I64, I, I, P, P, P, P, ctypes.c_size_t, P]
        L.svdq_w4a4_pack_weight.restype = I
        L.svdq_w4a4_prepare_workspace_bytes.argtypes = [I64, I64, I, I]
        L.svdq_w4a4_prepare_workspace_bytes.restype = ctypes.c_size_t
        L.svdq_w4a4_prepare_weight.argtypes = [P, P, I64, I64, I64, I, I, I, I, I, ctypes.c_uint64, P, P, P, P, P,
                                               P, P, P, ctypes.c_size_t, P]
        L.svdq_w4a4_prepare_weight.restype = I
        L.svdq_w4a4_gelu_table.argtypes = [P, P]
        L.svdq_w4a4_gelu_table.restype = I
        L.svdq_last_error.argtypes = []
        L.svdq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise SvdqError(rc, lib().svdq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _contig(t, dtype, name, shape=None):
    """Check one tensor argument before its pointer goes to the C ABI: its
    dtype, its shape (``shape`` a tuple, None entries match any size) and
    contiguity.  None passes through.  Raises ValueError naming the argument,
    so a caller's mistake cannot turn into an out-of-bounds device access.
    (That the tensors live on the GPU is checked by ``_on_gpu`` once every
    argument of a call has passed.)"""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(int(w)) for w in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(**tensors):
    """Every given tensor (None skipped) is a CUDA tensor."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")


def _workspace(ws, name="workspace"):
    return _contig(ws, torch.uint8, name, (None,))


def _out(out, M, N, device):
    """The bf16 [M, N] output: allocated if None, else checked."""
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    return _contig(out, torch.bfloat16, "out", (M, N))


def _x(x, K, name="x"):
    """A bf16 [M, K] activation matrix (K None: any width)."""
    return _contig(x, torch.bfloat16, name, (None, K))


def workspace_bytes(M, K, N, precision, rank):
    return lib().svdq_w4a4_workspace_bytes(M, K, N, PRECISIONS[precision], GROUP_SIZE[precision], rank)


class SVDQLinear:
    """Device-resident inputs of one svdq_w4a4 layer (all tensors on the GPU).

    packed_w uint8 [N, K/2]; wscales bf16 [N, K/64] (int4) or uint8 [N, K/16]
    (nvfp4); smooth bf16 [K]; lora_down bf16 [rank, K]; lora_up bf16 [N, rank];
    bias bf16 [N] or None; wtscale float (1.0 for int4).
    """

    def __init__(self, packed_w, wscales, smooth, lora_down, lora_up, bias, precision, wtscale=1.0):
        if precision not in PRECISIONS:
            raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
        self.precision = precision
        self.packed_w = _contig(packed_w, torch.uint8, "packed_w", (None, None))
        self.N, k2 = packed_w.shape
        self.K = 2 * k2
        if (lora_down is None) != (lora_up is None):
            raise ValueError("lora_down and lora_up must both be given or both be None")
        self.rank = 0 if lora_down is None else int(lora_down.shape[0])
        G = GROUP_SIZE[precision]
        if self.K % G:
            raise ValueError(f"K = {self.K} is not a multiple of the group size {G}")
        sdt = torch.bfloat16 if precision == "int4" else torch.uint8
        self.wscales = _contig(wscales, sdt, "wscales", (self.N, self.K // G))
        self.smooth = _contig(smooth, torch.bfloat16, "smooth", (self.K,))
        self.lora_down = _contig(lora_down, torch.bfloat16, "lora_down", (self.rank, self.K))
        self.lora_up = _contig(lora_up, torch.bfloat16, "lora_up", (self.N, self.rank))
        self.bias = _contig(bias, torch.bfloat16, "bias", (self.N,))
        self.wtscale = float(wtscale)
        _on_gpu(packed_w=self.packed_w, wscales=self.wscales, smooth=self.smooth, lora_down=self.lora_down,
                lora_up=self.lora_up, bias=self.bias)

    @classmethod
    def from_numpy(cls, d, device="cuda"):
        """From a dict of numpy arrays (bf16 tensors as uint16 bit patterns)."""
        def bf(a):
            if a is None:
                return None
            return torch.from_numpy(a.view("int16").copy()).view(torch.bfloat16).to(device)

        def u8(a):
            return torch.from_numpy(a.copy()).to(device)

        p = d["precision"]
        ws = bf(d["wscales"]) if p == "int4" else u8(d["wscales"])
        rank = d["rank"]
        return cls(u8(d["packed_w"]), ws, bf(d["smooth"]),
                   bf(d["lora_down"]) if rank else None, bf(d["lora_up"]) if rank else None,
                   bf(d.get("bias")), p, d.get("wtscale", 1.0))

    def workspace_bytes(self, M):
        return workspace_bytes(M, self.K, self.N, self.precision, self.rank)

    def __call__(self, x, out=None, workspace=None, stream=None):
        return svdq_w4a4_linear(x, self, out=out, workspace=workspace, stream=stream)


def svdq_w4a4_linear(x, layer, out=None, workspace=None, stream=None):
    """Y = svdq_w4a4(x) for a bf16 [M, K] CUDA tensor; returns bf16 [M, N]."""
    x = _x(x, layer.K)
    M, K = x.shape
    out = _out(out, M, layer.N, x.device)
    if workspace is None:
        workspace = torch.empty(max(layer.workspace_bytes(M), 1), dtype=torch.uint8, device=x.device)
    workspace = _workspace(workspace)
    _on_gpu(x=x, out=out, workspace=workspace)
    _check(lib().svdq_w4a4_linear(
        _ptr(x), M, K, layer.N, _ptr(layer.packed_w), _ptr(layer.wscales), layer.wtscale,
        _ptr(layer.smooth), _ptr(layer.lora_down), _ptr(layer.lora_up), _ptr(layer.bias),
        PRECISIONS[layer.precision], GROUP_SIZE[layer.precision], layer.rank, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # SVDQ_NOALLOC_SCRATCH_BYTES of include/svdq_w4a4.h


def svdq_w4a4_linear_noalloc(x, layer, out, stream=None):
    """svdq_w4a4_linear with the library's static device scratch instead of a
    workspace (for callers that cannot allocate: graph capture, serving loops);
    out is required (bf16 [M, N]).  Calls that overlap in time on one GPU race."""
    x = _x(x, layer.K)
    M, K = x.shape
    out = _contig(out, torch.bfloat16, "out", (M, layer.N))
    _on_gpu(x=x, out=out)
    _check(lib().svdq_w4a4_linear_noalloc(
        _ptr(x), M, K, layer.N, _ptr(layer.packed_w), _ptr(layer.wscales), layer.wtscale,
        _ptr(layer.smooth), _ptr(layer.lora_down), _ptr(layer.lora_up), _ptr(layer.bias),
        PRECISIONS[layer.precision], GROUP_SIZE[layer.precision], layer.rank, _ptr(out), _stream(stream)))
    return out


def svdq_w4a4_quantize(x, layer, workspace, stream=None):
    """First phase of svdq_w4a4_linear: quantize x into `workspace`."""
    x = _x(x, layer.K)
    M, K = x.shape
    workspace = _workspace(workspace)
    _on_gpu(x=x, workspace=workspace)
    _check(lib().svdq_w4a4_quantize(
        _ptr(x), M, K, _ptr(layer.smooth), _ptr(layer.lora_down), PRECISIONS[layer.precision],
        GROUP_SIZE[layer.precision], layer.rank, _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


def svdq_w4a4_gemm(workspace, M, layer, out=None, stream=None):
    """Second phase of svdq_w4a4_linear: the 4-bit product from `workspace`."""
    workspace = _workspace(workspace)
    out = _out(out, int(M), layer.N, workspace.device)
    _on_gpu(workspace=workspace, out=out)
    _check(lib().svdq_w4a4_gemm(
        _ptr(workspace), workspace.numel(), M, layer.K, layer.N, _ptr(layer.packed_w), _ptr(layer.wscales),
        layer.wtscale, _ptr(layer.lora_up), _ptr(layer.bias), PRECISIONS[layer.precision],
        GROUP_SIZE[layer.precision], layer.rank, _ptr(out), _stream(stream)))
    return out


def layer_struct(layer):
    """The svdq_w4a4_layer view of an SVDQLinear (pointers into its tensors)."""
    return LayerStruct(layer.packed_w.data_ptr(), layer.wscales.data_ptr(), layer.wtscale,
                       layer.smooth.data_ptr(), _addr(layer.lora_down), _addr(layer.lora_up), _addr(layer.bias),
                       layer.K, layer.N, PRECISIONS[layer.precision], GROUP_SIZE[layer.precision], layer.rank)


def _addr(t):
    return None if t is None else t.data_ptr()


def mlp_workspace_bytes(M, up, down):
    u, d = layer_struct(up), layer_struct(down)
    return lib().svdq_w4a4_mlp_workspace_bytes(M, ctypes.byref(u), ctypes.byref(d))


def svdq_w4a4_mlp_gelu(x, up, down, out=None, workspace=None, stream=None):
    """Y = down(GELU(up(x))) with the up projection's epilogue applying GELU and
    quantizing for the down projection (nvfp4 down layer); returns bf16 [M, N_down]."""
    if up.N != down.K:
        raise ValueError(f"the up layer's N ({up.N}) must equal the down layer's K ({down.K})")
    x = _x(x, up.K)
    M = x.shape[0]
    u, d = layer_struct(up), layer_struct(down)
    out = _out(out, M, down.N, x.device)
    if workspace is None:
        need = lib().svdq_w4a4_mlp_workspace_bytes(M, ctypes.byref(u), ctypes.byref(d))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    workspace = _workspace(workspace)
    _on_gpu(x=x, out=out, workspace=workspace)
    _check(lib().svdq_w4a4_mlp_gelu(_ptr(x), M, ctypes.byref(u), ctypes.byref(d), _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))
    return out


def svdq_w4a4_qkv_rmsnorm_rope(x, qkv, heads, q_norm, k_norm, rope_cos, rope_sin, eps=1e-6, out=None,
                               workspace=None, stream=None):
    """Fused QKV projection: q | k | v = qkv(x) with per-head RMSNorm (weights
    q_norm / k_norm, bf16 [D]; the head dim D = 32, 64 or 128 is their
    length) and RoPE (rope_cos / rope_sin, fp32 [M, D/2], interleaved pairs)
    applied to the q and k heads in the projection's epilogue; returns bf16
    [M, 3 heads D]."""
    x = _x(x, qkv.K)
    M = x.shape[0]
    q = layer_struct(qkv)
    q_norm = _contig(q_norm, torch.bfloat16, "q_norm", (None,))
    head_dim = q_norm.numel()
    k_norm = _contig(k_norm, torch.bfloat16, "k_norm", (head_dim,))
    rope_cos = _contig(rope_cos, torch.float32, "rope_cos", (M, head_dim // 2))
    rope_sin = _contig(rope_sin, torch.float32, "rope_sin", (M, head_dim // 2))
    out = _out(out, M, qkv.N, x.device)
    if workspace is None:
        workspace = torch.empty(max(qkv.workspace_bytes(M), 1), dtype=torch.uint8, device=x.device)
    workspace = _workspace(workspace)
    _on_gpu(x=x, q_norm=q_norm, k_norm=k_norm, rope_cos=rope_cos, rope_sin=rope_sin, out=out, workspace=workspace)
    _check(lib().svdq_w4a4_qkv_rmsnorm_rope(
        _ptr(x), M, ctypes.byref(q), heads, head_dim, _ptr(q_norm), _ptr(k_norm), float(eps), _ptr(rope_cos),
        _ptr(rope_sin), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def gelu_table(stream=None):
    """Parity export: the fused MLP epilogue's bf16 GELU table, uint16 [65536]
    (entry b = bf16 bits of GELU of the bf16 value with bits b)."""
    out = torch.empty(1 << 16, dtype=torch.int16, device="cuda")
    _check(lib().svdq_w4a4_gelu_table(_ptr(out), _stream(stream)))
    return out


# ---- offline weight preparation on the GPU -----------------------------------------
def _prep_ws(K, workspace, device):
    if workspace is None:
        workspace = torch.empty(max(lib().svdq_w4a4_prep_workspace_bytes(K), 1), dtype=torch.uint8, device=device)
    return _workspace(workspace)


def smooth_factors(x_calib, w, workspace=None, stream=None):
    """bf16 [K] smoothing factors sqrt(max|x| / max|w|) per input channel of a
    weight w (fp32 [N, K]) from calibration activations x_calib (bf16 [M, K])."""
    w = _contig(w, torch.float32, "w", (None, None))
    x_calib = _contig(x_calib, torch.bfloat16, "x_calib", (None, w.shape[1]))
    (M, K), N = x_calib.shape, w.shape[0]
    out = torch.empty(K, dtype=torch.bfloat16, device=w.device)
    workspace = _prep_ws(K, workspace, w.device)
    _on_gpu(x_calib=x_calib, w=w, workspace=workspace)
    _check(lib().svdq_w4a4_smooth_factors(_ptr(x_calib), M, _ptr(w), N, K, _ptr(out), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return out


def pack_weight(resid, precision, workspace=None, stream=None):
    """Quantize and pack a residual weight (fp32 [N, K]): returns (packed_w
    uint8 [N, K/2], wscales, wtscale as a 1-element fp32 device tensor)."""
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    resid = _contig(resid, torch.float32, "resid", (None, None))
    N, K = resid.shape
    G = GROUP_SIZE[precision]
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=resid.device)
    wscales = torch.empty((N, K // G), dtype=torch.bfloat16 if precision == "int4" else torch.uint8,
                          device=resid.device)
    wt = torch.empty(4, dtype=torch.float32, device=resid.device)
    workspace = _prep_ws(K, workspace, resid.device)
    _on_gpu(resid=resid, workspace=workspace)
    _check(lib().svdq_w4a4_pack_weight(_ptr(resid), N, K, PRECISIONS[precision], G, _ptr(packed), _ptr(wscales),
                                       _ptr(wt), _ptr(workspace), workspace.numel(), _stream(stream)))
    return packed, wscales, wt[:1]


def prepare_layer(w, x_calib, rank, precision, bias=None, oversample=16, power_iters=6, seed=0,
                  workspace=None, stream=None, return_sigma=False):
    """A ready SVDQLinear from a weight (fp32 [N, K] CUDA tensor) and
    calibration activations (bf16 [M, K]), prepared on the GPU by
    svdq_w4a4_prepare_weight: smoothing factors, the rank-r split of the
    smoothed weight (randomized range finder with subspace iteration), and the
    residual's quantization and packing.  Offline: the call synchronizes.
    With return_sigma, also returns the estimated leading singular values."""
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    w = _contig(w, torch.float32, "w", (None, None))
    N, K = w.shape
    x_calib = _x(x_calib, K, "x_calib")
    bias = _contig(bias, torch.bfloat16, "bias", (N,))
    G = GROUP_SIZE[precision]
    dev = w.device
    smooth = torch.empty(K, dtype=torch.bfloat16, device=dev)
    down = torch.empty((rank, K), dtype=torch.bfloat16, device=dev) if rank else None
    up = torch.empty((N, rank), dtype=torch.bfloat16, device=dev) if rank else None
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    wscales = torch.empty((N, K // G), dtype=torch.bfloat16 if precision == "int4" else torch.uint8, device=dev)
    wt = torch.empty(4, dtype=torch.float32, device=dev)
    if workspace is None:
        need = lib().svdq_w4a4_prepare_workspace_bytes(N, K, rank, oversample)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    workspace = _workspace(workspace)
    _on_gpu(w=w, x_calib=x_calib, bias=bias, workspace=workspace)
    sigma = (ctypes.c_double * max(rank, 1))()
    _check(lib().svdq_w4a4_prepare_weight(
        _ptr(w), _ptr(x_calib), x_calib.shape[0], N, K, PRECISIONS[precision], G, rank, oversample, power_iters,
        int(seed) & (2 ** 64 - 1), _ptr(smooth), _ptr(down), _ptr(up), _ptr(packed), _ptr(wscales), _ptr(wt),
        sigma, _ptr(workspace), workspace.numel(), _stream(stream)))
    layer = SVDQLinear(packed, wscales, smooth, down, up, bias, precision, float(wt[0].item()))
    if return_sigma:
        return layer, [sigma[i] for i in range(rank)]
    return layer


class AWQLinear:
    """Device-resident inputs of one awq_w4a16 layer: packed_w uint8 [N, K/2],
    wscales / wzeros bf16 [N, K/64], bias bf16 [N] or None."""

    def __init__(self, packed_w, wscales, wzeros, bias=None):
        self.packed_w = _contig(packed_w, torch.uint8, "packed_w", (None, None))
        self.N, k2 = packed_w.shape
        self.K = 2 * k2
        if self.K % 64:
            raise ValueError(f"K = {self.K} is not a multiple of the group size 64")
        self.wscales = _contig(wscales, torch.bfloat16, "wscales", (self.N, self.K // 64))
        self.wzeros = _contig(wzeros, torch.bfloat16, "wzeros", (self.N, self.K // 64))
        self.bias = _contig(bias, torch.bfloat16, "bias", (self.N,))
        _on_gpu(packed_w=self.packed_w, wscales=self.wscales, wzeros=self.wzeros, bias=self.bias)

    @classmethod
    def from_numpy(cls, d, device="cuda"):
        def bf(a):
            if a is None:
                return None
            return torch.from_numpy(a.view("int16").copy()).view(torch.bfloat16).to(device)
        return cls(torch.from_numpy(d["packed_w"].copy()).to(device), bf(d["wscales"]),
                   bf(d["wzeros"]), bf(d.get("bias")))

    def __call__(self, x, out=None, stream=None):
        return awq_w4a16_linear(x, self, out=out, stream=stream)


def awq_w4a16_linear(x, layer, out=None, stream=None):
    """Y = awq_w4a16(x) for a bf16 [M, K] CUDA tensor; returns bf16 [M, N]."""
    x = _x(x, layer.K)
    M, K = x.shape
    out = _out(out, M, layer.N, x.device)
    _on_gpu(x=x, out=out)
    _check(lib().awq_w4a16_linear(
        _ptr(x), M, K, layer.N, _ptr(layer.packed_w), _ptr(layer.wscales), _ptr(layer.wzeros),
        _ptr(layer.bias), 64, _ptr(out), _stream(stream)))
    return out


def svdq_w4a4_quantize_act(x, smooth, lora_down, precision, stream=None, out=None):
    """Kernel 1 on its own: returns (codes uint8 [M, K/2], scales, lora_act fp32 [M, rank]).
    ``out`` may pass preallocated (codes, scales, lora_act) tensors."""
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    x = _x(x, None)
    M, K = x.shape
    smooth = _contig(smooth, torch.bfloat16, "smooth", (K,))
    lora_down = _contig(lora_down, torch.bfloat16, "lora_down", (None, K))
    rank = 0 if lora_down is None else lora_down.shape[0]
    G = GROUP_SIZE[precision]
    sdt = torch.bfloat16 if precision == "int4" else torch.uint8
    if out is not None:
        codes, scales, lora_act = out
        codes = _contig(codes, torch.uint8, "codes", (M, K // 2))
        scales = _contig(scales, sdt, "scales", (M, K // G))
        lora_act = _contig(lora_act, torch.float32, "lora_act", (M, rank))
    else:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((M, K // G), dtype=sdt, device=x.device)
        lora_act = torch.empty((M, rank), dtype=torch.float32, device=x.device) if rank else None
    _on_gpu(x=x, smooth=smooth, lora_down=lora_down, codes=codes, scales=scales, lora_act=lora_act)
    _check(lib().svdq_w4a4_quantize_act(
        _ptr(x), M, K, _ptr(smooth), _ptr(lora_down), PRECISIONS[precision], G, rank,
        _ptr(codes), _ptr(scales), _ptr(lora_act), _stream(stream)))
    return codes, scales, lora_act


def svdq_w4a4_quantize_operand(x, smooth, lora_down, precision, stream=None):
    """Kernel 1 exactly as the linear launches it: returns (operand, scale,
    lora_act fp32 [M, rank] or None) -- int4: operand uint8 [M, K], the codes
    as fp8 E4M3 bytes, and scale fp32 [M, K/64], the group scales; nvfp4:
    operand float16 [M, K], e2m1 * dec(s8), and scale None."""
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    x = _x(x, None)
    M, K = x.shape
    smooth = _contig(smooth, torch.bfloat16, "smooth", (K,))
    lora_down = _contig(lora_down, torch.bfloat16, "lora_down", (None, K))
    rank = 0 if lora_down is None else lora_down.shape[0]
    int4 = precision == "int4"
    operand = torch.empty((M, K), dtype=torch.uint8 if int4 else torch.float16, device=x.device)
    scale = torch.empty((M, K // 64), dtype=torch.float32, device=x.device) if int4 else None
    lora_act = torch.empty((M, rank), dtype=torch.float32, device=x.device) if rank else None
    _on_gpu(x=x, smooth=smooth, lora_down=lora_down)
    _check(lib().svdq_w4a4_quantize_operand(
        _ptr(x), M, K, _ptr(smooth), _ptr(lora_down), PRECISIONS[precision], GROUP_SIZE[precision], rank,
        _ptr(operand), _ptr(scale), _ptr(lora_act), _stream(stream)))
    return operand, scale, lora_act


def svdq_w4a4_gemm_partials(act_codes, w_codes, precision, stream=None):
    """Parity export of kernel 2's 4-bit product: int32 [M, N, K/G]."""
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    act_codes = _contig(act_codes, torch.uint8, "act_codes", (None, None))
    w_codes = _contig(w_codes, torch.uint8, "w_codes", (None, act_codes.shape[1]))
    M, k2 = act_codes.shape
    N = w_codes.shape[0]
    K = 2 * k2
    G = GROUP_SIZE[precision]
    out = torch.empty((M, N, K // G), dtype=torch.int32, device=act_codes.device)
    _on_gpu(act_codes=act_codes, w_codes=w_codes)
    _check(lib().svdq_w4a4_gemm_partials(
        _ptr(act_codes), _ptr(w_codes), M, K, N, PRECISIONS[precision], G, _ptr(out), _stream(stream)))
    return out
