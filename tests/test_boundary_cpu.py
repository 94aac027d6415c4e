"""C-ABI boundary on the CPU: the library loads without a GPU, exports every
entry point of include/svdq_w4a4.h, and its host-side validation returns the
documented status for every class of bad argument (no device memory is ever
touched: the pointers below are fake, aligned addresses)."""

import ctypes
import json
import os
import re

import pytest

import bit_quantized_linear_quantize_amd as bq
from split_rule import k1_slices, ksplit, lora_part_bytes, split_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq_w4a4.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

OK, EINVAL, EUNSUP, EARCH, EWS, EDEV = 0, -1, -2, -3, -4, -5
GFX950 = b"gfx950:sramecc+:xnack-"


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bq.LIB_PATH):
        from bit_quantized_linear_quantize_amd import build
        build.build()
    return bq.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s+([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported(L):
    names = header_functions()
    assert set(names) == set(bq.EXPORTS), names
    for n in names:
        assert getattr(L, n) is not None


def test_peak_probe_library_exports(L):
    # the benchmark helper (measured matrix-instruction peak) is its own library
    path = os.path.join(os.path.dirname(bq.LIB_PATH), "libsvdq_peak.so")
    assert os.path.exists(path)
    assert ctypes.CDLL(path).svdq_peak_mfma_f16 is not None


def _fake(base):
    return ctypes.c_void_p(base)


class Args:
    """A valid svdq_w4a4 call (fake, disjoint, aligned pointers)."""

    def __init__(self, M=256, K=512, N=256, precision=0, group=64, rank=32):
        self.M, self.K, self.N = M, K, N
        self.precision, self.group, self.rank = precision, group, rank
        self.x = 0x1000_0000
        self.w = 0x2000_0000
        self.ws = 0x3000_0000
        self.sm = 0x4000_0000
        self.ld = 0x5000_0000
        self.lu = 0x6000_0000
        self.b = 0x7000_0000
        self.out = 0x8000_0000
        self.work = 0x9000_0000
        self.wt = 1.0 if precision == 0 else 0.01
        self.wsb = None

    def call(self, L, arch=GFX950, **kw):
        d = dict(vars(self))
        d.update(kw)
        wsb = d["wsb"]
        if wsb is None:
            wsb = L.svdq_w4a4_workspace_bytes(d["M"], d["K"], d["N"], d["precision"], d["group"], d["rank"])
        p = lambda v: None if v is None else _fake(v)
        return L.svdq_w4a4_check(p(d["x"]), d["M"], d["K"], d["N"], p(d["w"]), p(d["ws"]), d["wt"],
                                 p(d["sm"]), p(d["ld"]), p(d["lu"]), p(d["b"]), d["precision"],
                                 d["group"], d["rank"], p(d["out"]), p(d["work"]), wsb, arch)


def test_valid_calls_pass(L):
    assert Args().call(L) == OK
    assert Args(precision=1, group=16).call(L) == OK
    assert Args(rank=0).call(L, ld=None, lu=None) == OK
    assert Args().call(L, b=None) == OK
    assert Args(M=1, K=128, N=64).call(L) == OK


def test_only_the_tabled_precision_group_pairs(L):
    tab = json.load(open(os.path.join(GOLDEN, "quantization_types.json")))
    legal = {(bq.PRECISIONS[r["precision"]], r["group_size"]) for r in tab["rows"] if r["method"] == "svdq_w4a4"}
    for prec in (0, 1, 2, -1):
        for g in (8, 16, 32, 64, 128):
            rc = Args(precision=prec if prec in (0, 1) else 0, group=g).call(L, precision=prec, group=g,
                                                                               wt=1.0 if prec != 1 else 0.01)
            assert (rc == OK) == ((prec, g) in legal), (prec, g, rc)
            if (prec, g) not in legal:
                assert rc == EUNSUP


def test_rank_bounds(L):
    for r, want in ((0, OK), (16, OK), (32, OK), (128, OK), (8, EUNSUP), (144, EUNSUP), (-16, EUNSUP)):
        kw = {} if r else dict(ld=None, lu=None)
        assert Args(rank=r).call(L, rank=r, **kw) == want, r


def test_shape_rules(L):
    assert Args().call(L, M=0) == EINVAL
    assert Args().call(L, K=192) == EINVAL
    assert Args().call(L, K=64) == EINVAL
    assert Args().call(L, N=96) == EINVAL
    assert Args().call(L, K=32768) == EINVAL
    # the product kernel's grid: at most 2^23 - 1 tiles of 256 x 192
    M = 1 << 24
    assert L.svdq_w4a4_workspace_bytes(M, 512, 127 * 192, 0, 64, 32) > 0
    assert L.svdq_w4a4_workspace_bytes(M, 512, 128 * 192, 0, 64, 32) == 0
    assert Args().call(L, M=M, N=128 * 192, wsb=1 << 62) == EINVAL
    assert b"output tiles" in L.svdq_last_error()


def test_null_and_alignment(L):
    for f in ("x", "w", "ws", "sm", "out", "work"):
        assert Args().call(L, **{f: None}) == EINVAL, f
    assert Args().call(L, ld=None) == EINVAL
    assert Args(rank=0).call(L, rank=0) == EINVAL  # lora given with rank 0
    for f in ("x", "w", "ws", "sm", "ld", "lu", "b", "out", "work"):
        a = Args()
        assert a.call(L, **{f: getattr(a, f) + 8}) == EINVAL, f


def test_aliasing(L):
    a = Args()
    assert a.call(L, out=a.x) == EINVAL
    assert a.call(L, out=a.x + 1024) == EINVAL
    assert a.call(L, out=a.work) == EINVAL
    assert a.call(L, out=a.w + 64) == EINVAL


def test_wtscale_rules(L):
    assert Args().call(L, wt=0.5) == EINVAL
    assert Args(precision=1, group=16).call(L, wt=0.0) == EINVAL
    assert Args(precision=1, group=16).call(L, wt=float("inf")) == EINVAL


def test_split_rule():
    assert ksplit(4096, 3072, 3072) == 1          # 256 tiles
    assert ksplit(2048, 3072, 3072) == 2          # 128 tiles: half the compute units
    assert ksplit(2048, 3264, 3072) == 1          # 136 tiles
    assert ksplit(512, 3072, 3072) == 8           # 32 tiles
    assert ksplit(1024, 3072, 3072) == 4          # 64 tiles
    assert ksplit(300, 320, 512) == 2             # 4 tiles, 8 stages: at most max(2, 8 // 5) splits
    assert ksplit(64, 64, 128) == 1               # 2 stages
    assert ksplit(64, 64, 576) == 2               # 9 stages
    assert ksplit(64, 64, 1152) == 3              # 18 stages
    assert ksplit(256, 3072, 960) == 3            # 15 stages: 15 // 5 = 3 splits of 5
    assert ksplit(64, 128, 3200) == 8             # 50 stages: 7 splits of 7, the last of 1
    # int4 stages are 128 values of K
    assert ksplit(512, 3072, 3072, "int4") == 4   # 24 stages: about five per split
    assert ksplit(512, 3072, 6144, "int4") == 8   # 48 stages
    assert ksplit(300, 320, 512, "int4") == 2     # 4 stages
    assert ksplit(64, 64, 256, "int4") == 1       # 2 stages
    assert ksplit(64, 64, 1152, "int4") == 2      # 9 stages
    assert ksplit(64, 128, 3200, "int4") == 5     # 25 stages: 5 splits of 5


def test_workspace_size(L):
    M, K, N = 300, 512, 320
    rnd = lambda v: (v + 255) // 256 * 256
    # the product operand (int4: fp8 codes [M, K] and bf16 group scales
    # [M, K/64]; nvfp4: fp16 [M, K]); then lora_act fp32 [M, 32]; then, with
    # kernel 1 split along K, its low-rank slice partials fp32 [S, M, 32];
    # then the split-K partials fp32 [ksplit, M, N]
    assert k1_slices(M, K) == 8 and k1_slices(4096, 3072) == 1 and k1_slices(2048, 3072) == 2
    assert k1_slices(512, 3072) == 8 and k1_slices(64, 384) == 2 and k1_slices(1, 128) == 2
    want = {0: rnd(M * K) + rnd(2 * M * (K // 64)) + rnd(M * 32 * 4) + lora_part_bytes(M, K, 32) +
            split_bytes(M, N, K, "int4"),
            1: rnd(2 * M * K) + rnd(M * 32 * 4) + lora_part_bytes(M, K, 32) + split_bytes(M, N, K)}
    assert split_bytes(M, N, K) > 0 and split_bytes(M, N, K, "int4") > 0
    assert L.svdq_w4a4_workspace_bytes(4096, 3072, 3072, 1, 16, 32) == rnd(2 * 4096 * 3072) + rnd(4096 * 32 * 4)
    for prec, g in ((0, 64), (1, 16)):
        need = L.svdq_w4a4_workspace_bytes(M, K, N, prec, g, 32)
        assert need == want[prec]
        a = Args(M=M, K=K, N=N, precision=prec, group=g)
        assert a.call(L, wsb=need - 1) == EWS
        assert a.call(L, wsb=need) == OK
    assert L.svdq_w4a4_workspace_bytes(M, K, N, 0, 16, 32) == 0


def test_arch_rule(L):
    assert Args().call(L, arch=b"gfx942:sramecc+:xnack-") == EARCH
    assert Args().call(L, arch=b"gfx1100") == EARCH
    assert Args().call(L, arch=GFX950) == OK


def test_error_message(L):
    Args().call(L, K=192)
    assert b"K must be" in L.svdq_last_error()
    Args().call(L)
    assert L.svdq_last_error() == b""


def test_awq_rules(L):
    p = _fake
    def call(M=16, K=3072, N=18432, x=0x1000_0000, w=0x2000_0000, s=0x3000_0000, z=0x4000_0000,
             b=0x5000_0000, g=64, out=0x8000_0000, arch=GFX950):
        q = lambda v: None if v is None else p(v)
        return L.awq_w4a16_check(q(x), M, K, N, q(w), q(s), q(z), q(b), g, q(out), arch)
    assert call() == OK
    assert call(b=None) == OK
    assert call(g=128) == EUNSUP
    assert call(K=100) == EINVAL
    assert call(z=None) == EINVAL
    assert call(out=0x1000_0000 + 64) == EINVAL
    assert call(arch=b"gfx90a") == EARCH
    assert call(x=0x1000_0004) == EINVAL


def test_linear_rejects_before_touching_the_device(L):
    # validation runs first: an unsupported pair never reaches the HIP runtime
    rc = L.svdq_w4a4_linear(_fake(0x1000_0000), 256, 512, 256, _fake(0x2000_0000), _fake(0x3000_0000),
                            1.0, _fake(0x4000_0000), None, None, None, 0, 32, 0, _fake(0x8000_0000),
                            _fake(0x9000_0000), 1 << 20, None)
    assert rc == EUNSUP


def test_operand_export_rejects_before_touching_the_device(L):
    # svdq_w4a4_quantize_operand validates everything before its device check
    def call(prec=0, group=64, rank=16, rs=0x3000_0000, la=0x4000_0000, op=0x2000_0000, ld=0x5000_0000,
             M=64, K=512):
        return L.svdq_w4a4_quantize_operand(_fake(0x1000_0000), M, K, _fake(0x6000_0000),
                                            None if ld is None else _fake(ld), prec, group, rank,
                                            None if op is None else _fake(op), None if rs is None else _fake(rs),
                                            None if la is None else _fake(la), None)
    assert call(group=16) == EUNSUP
    assert call(rank=24) == EUNSUP
    assert call(K=100) == EINVAL
    assert call(rs=None) == EINVAL              # int4 needs the row factors
    assert call(prec=1, group=16) == EINVAL     # nvfp4 has none
    assert call(la=None) == EINVAL
    assert call(ld=None) == EINVAL
    assert call(op=None) == EINVAL
    assert call(op=0x1000_0000 + 64) == EINVAL  # overlaps x
    assert call(rs=0x2000_0000 + 256) == EINVAL  # overlaps the operand
    assert call(op=0x2000_0008) == EINVAL       # misaligned


# ------------------------------------------------------------------ fused GELU MLP
def _layer(base, K, N, precision=1, rank=32, wt=None):
    group = 16 if precision == 1 else 64
    wt = (1.0 if precision == 0 else 0.01) if wt is None else wt
    return bq.LayerStruct(base, base + 0x100_0000, wt, base + 0x200_0000,
                          base + 0x300_0000 if rank else None, base + 0x400_0000 if rank else None,
                          base + 0x500_0000, K, N, precision, group, rank)


def test_mlp_rules(L):
    M, K, H, N = 256, 512, 768, 256
    x, out, ws = 0x3_0000_0000, 0x4_0000_0000, 0x5_0000_0000
    up, down = _layer(0x1_0000_0000, K, H, precision=0), _layer(0x2_0000_0000, H, N, precision=1)
    B = ctypes.byref
    need = L.svdq_w4a4_mlp_workspace_bytes(M, B(up), B(down))
    rnd = lambda v: (v + 255) // 256 * 256
    # the up layer's operand (int4: fp8 codes and bf16 group scales) and
    # lora_act, the down layer's linear workspace, then the down layer's
    # low-rank partials per 192-column tile of the up projection
    assert need == (rnd(M * K) + rnd(2 * M * (K // 64)) + rnd(4 * M * 32) + lora_part_bytes(M, K, 32)) + \
        (rnd(2 * M * H) + rnd(4 * M * 32) + lora_part_bytes(M, H, 32) + split_bytes(M, N, H)) + \
        rnd(4 * ((H + 191) // 192) * M * 32)

    def call(x=x, M=M, up=up, down=down, out=out, ws=ws, wsb=need, arch=GFX950):
        p = lambda v: None if v is None else _fake(v)
        return L.svdq_w4a4_mlp_gelu_check(p(x), M, B(up) if up is not None else None,
                                          B(down) if down is not None else None, p(out), p(ws), wsb, arch)
    assert call() == OK
    up_n = _layer(0x1_0000_0000, K, H, precision=1)  # an nvfp4 up layer keeps an fp16 operand
    need_n = L.svdq_w4a4_mlp_workspace_bytes(M, B(up_n), B(down))
    assert need_n == need + rnd(2 * M * K) - rnd(M * K) - rnd(2 * M * (K // 64))
    assert call(up=up_n, wsb=need_n) == OK and call(up=up_n) == EWS
    assert call(down=_layer(0x2_0000_0000, H, N, precision=0)) == EUNSUP  # int4 hidden activations
    assert L.svdq_w4a4_mlp_workspace_bytes(M, B(up), B(_layer(0x2_0000_0000, H, N, precision=0))) == 0
    assert call(down=_layer(0x2_0000_0000, H + 64, N)) == EINVAL     # up->N != down->K
    assert call(up=None) == EINVAL
    assert call(wsb=need - 1) == EWS
    assert call(x=x + 8) == EINVAL
    assert call(out=ws) == EINVAL                                     # out overlaps the workspace
    assert call(down=_layer(0x2_0000_0000, H, N, rank=0)) == OK
    assert call(down=_layer(0x2_0000_0000, H, N, rank=24)) == EUNSUP
    assert call(arch=b"gfx942") == EARCH


def test_qkv_rules(L):
    M, K, H = 256, 512, 4
    N = 3 * H * 128
    x, out, ws = 0x3_0000_0000, 0x4_0000_0000, 0x5_0000_0000
    qn, kn, cs, sn = 0x6_0000_0000, 0x6_0001_0000, 0x7_0000_0000, 0x8_0000_0000
    qkv = _layer(0x1_0000_0000, K, N, precision=1)
    B = ctypes.byref
    # the linear's activations, lora_act and kernel 1's low-rank slice
    # partials (no split partials: the epilogue is not split)
    need = (2 * M * K + 255) // 256 * 256 + (M * 32 * 4 + 255) // 256 * 256 + lora_part_bytes(M, K, 32)

    def call(x=x, M=M, qkv=qkv, heads=H, hd=128, qn=qn, kn=kn, eps=1e-6, cs=cs, sn=sn, out=out, ws=ws,
             wsb=need, arch=GFX950):
        p = lambda v: None if v is None else _fake(v)
        return L.svdq_w4a4_qkv_rmsnorm_rope_check(p(x), M, B(qkv) if qkv is not None else None, heads, hd, p(qn),
                                                  p(kn), eps, p(cs), p(sn), p(out), p(ws), wsb, arch)
    assert call() == OK
    assert call(qkv=_layer(0x1_0000_0000, K, N, precision=0), wsb=need + (4 * M + 255) // 256 * 256) == OK
    assert call(hd=64) == EINVAL                    # N != 3 heads head_dim
    assert call(hd=64, heads=8) == OK               # head dims 32, 64 and 128
    assert call(hd=32, heads=16) == OK
    for hd in (16, 48, 96, 256):                    # other head dims
        assert call(hd=hd, heads=N // (3 * hd)) == EUNSUP
    assert call(hd=256, heads=2) == EUNSUP
    assert call(heads=3) == EINVAL                  # N != 3 heads head_dim
    assert call(heads=0) == EINVAL
    big = 257
    assert call(heads=big, qkv=_layer(0x1_0000_0000, K, 3 * big * 128)) == EINVAL
    for e in (0.0, -1e-6, float("nan"), float("inf")):
        assert call(eps=e) == EINVAL
    assert call(qn=None) == EINVAL and call(kn=None) == EINVAL
    assert call(cs=None) == EINVAL and call(sn=None) == EINVAL
    assert call(cs=cs + 8) == EINVAL                # alignment
    assert call(out=sn) == EINVAL                   # out overlaps a table
    assert call(out=ws) == EINVAL                   # out overlaps the workspace
    assert call(wsb=need - 1) == EWS
    assert call(qkv=_layer(0x1_0000_0000, K, N, rank=24)) == EUNSUP
    assert call(qkv=None) == EINVAL
    assert call(arch=b"gfx942") == EARCH


def test_prep_rules(L):
    K, M, N = 1024, 64, 384
    x, w, sm, ws = 0x1_0000_0000, 0x2_0000_0000, 0x3_0000_0000, 0x4_0000_0000
    need = L.svdq_w4a4_prep_workspace_bytes(K)
    assert need == 8 * K and L.svdq_w4a4_prep_workspace_bytes(0) == 0
    p = lambda v: None if v is None else _fake(v)

    def smooth(x=x, M=M, w=w, N=N, K=K, sm=sm, ws=ws, wsb=need):
        return L.svdq_w4a4_smooth_factors(p(x), M, p(w), N, K, p(sm), p(ws), wsb, None)
    # (argument errors are found before the device is queried)
    assert smooth(M=0) == EINVAL and smooth(N=(1 << 22) + 1) == EINVAL
    assert smooth(K=1000) == EINVAL
    assert smooth(x=None) == EINVAL and smooth(sm=None) == EINVAL
    assert smooth(w=w + 4) == EINVAL
    assert smooth(sm=w + 64) == EINVAL                 # output inside w
    assert smooth(wsb=need - 1) == EWS

    r, pk, sc, wt = 0x5_0000_0000, 0x6_0000_0000, 0x7_0000_0000, 0x8_0000_0000

    def pack(r=r, N=N, K=K, prec=1, G=16, pk=pk, sc=sc, wt=wt, ws=ws, wsb=need):
        return L.svdq_w4a4_pack_weight(p(r), N, K, prec, G, p(pk), p(sc), p(wt), p(ws), wsb, None)
    assert pack(G=64) == EUNSUP and pack(prec=0, G=16) == EUNSUP and pack(prec=2) == EUNSUP
    assert pack(K=100) == EINVAL and pack(N=0) == EINVAL
    assert pack(wt=None) == EINVAL                     # nvfp4 needs the tensor scale output
    assert pack(wt=wt + 2) == EINVAL
    assert pack(pk=r) == EINVAL                        # output overlaps the residual
    assert pack(sc=pk + 16) == EINVAL                  # outputs overlap
    assert pack(wsb=0) == EWS
