"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars:
* activation codes, activation scales and per-group integer partials: bit-exact;
* low-rank activations (fp32): max |err| <= 1e-4 * max |ref|;
* bf16 output Y against the fp64 oracle:
    max(|err| - half a bf16 ulp of Y_ref) <= 1e-2 * RMS(Y_ref), and
    mean relative error sum|err| / sum|Y_ref| <= 2e-3 (rounding included).
  The first bar does not charge the final rounding to the bf16 output dtype
  to the kernel: with outlier channels |Y| reaches many times RMS(Y), and half
  a bf16 ulp of such an element alone exceeds 1e-2 * RMS(Y), so no bf16 result
  could meet a bound on the raw error.  What remains (fp32 accumulation order,
  the bf16 hi/lo split of the low-rank operands) must stay within the bound.
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F, layers as L, quant as Q
from exact_mlp import exact_up_problem
from split_rule import ksplit
import tie_inputs as T

pytestmark = pytest.mark.gpu

bq = pytest.importorskip("bit_quantized_linear_quantize_amd")


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a).copy()).cuda()


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ones_smooth(K):
    return F.bf16_bits(np.ones(K, np.float32))


def assert_output(y_dev, y_ref, label):
    y = F.bf16_to_f32(host_bits(y_dev)).astype(np.float64)
    maxrel, excess, mre = L.output_errors(y, y_ref)
    print(f"[{label}] max|err|/RMS={maxrel:.3e} (beyond half-ulp {excess:.3e}) MRE={mre:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert excess <= 1e-2, label
    assert mre <= 2e-3, label


def prepared(x, w, bias, precision, rank, smooth="ones"):
    K = w.shape[1]
    sm = ones_smooth(K) if smooth == "ones" else L.smooth_factors(x, w)
    return L.prepare_svdq_layer(w, sm, rank, precision, bias)


def run_linear(x_bits, lay, poison=None):
    layer = bq.SVDQLinear.from_numpy(lay)
    x = dev_bf16(x_bits)
    ws = torch.empty(max(layer.workspace_bytes(x.shape[0]), 1), dtype=torch.uint8, device="cuda")
    if poison is not None:
        ws.fill_(poison)
    y = layer(x, workspace=ws)
    torch.cuda.synchronize()
    return y


# ------------------------------------------------------------------ fixtures
@pytest.fixture(scope="module")
def cfg0():
    c = S.config0()
    return c


@pytest.fixture(scope="module")
def ragged():
    rng = np.random.default_rng(11)
    M, K, N = 300, 512, 320
    x = S.activations(M, K, 5, rng)
    w = S.weight(N, K, 0.02, rng, spike_rank=4)
    b = S.bias(N, rng)
    return x, w, b


@pytest.fixture(scope="module")
def cfg1_layers():
    c = S.config1()
    sm = L.smooth_factors(c["x"], c["w"])
    lay4 = L.prepare_svdq_layer(c["w"], sm, 32, "int4", c["bias"])
    lay_fp4 = L.prepare_svdq_layer(c["w"], sm, 32, "nvfp4", c["bias"])
    return c, lay4, lay_fp4


# ------------------------------------------------------------------ kernel 1
def check_quantize_act(x_bits, lay, label):
    p = lay["precision"]
    ref = L.svdq_quantize_act(x_bits, lay["smooth"], lay["lora_down"], p)
    x = dev_bf16(x_bits)
    ld = dev_bf16(lay["lora_down"]) if lay["rank"] else None
    codes, scales, lora = bq.svdq_w4a4_quantize_act(x, dev_bf16(lay["smooth"]), ld, p)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    sc = host_bits(scales) if p == "int4" else scales.cpu().numpy()
    bad = np.argwhere(codes != ref["packed"])
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first {bad[:4].tolist()}"
    assert np.array_equal(sc, ref["scales"]), f"{label}: scales differ"
    if lay["rank"]:
        la = lora.cpu().numpy().astype(np.float64)
        err = np.abs(la - ref["lora_act"]).max()
        tol = 1e-4 * np.abs(ref["lora_act"]).max() + 1e-6
        print(f"[{label}] lora_act max err {err:.3e} (tol {tol:.3e})", flush=True)
        assert err <= tol, label


def check_operand(x_bits, lay, label):
    """The first kernel as the linear launches it (svdq_w4a4_quantize_operand)
    against the oracle: int4 the E4M3 code bytes and the fp32 group scales bit
    for bit; nvfp4 the binary16 operand value for value (exact equality, so +0
    and -0 agree); the low-rank activations to 1e-4 of their largest
    magnitude."""
    p = lay["precision"]
    ref = L.svdq_quantize_act(x_bits, lay["smooth"], lay["lora_down"], p)
    want, want_sc = L.product_operand_ref(ref["codes"], ref["scales"], p)
    ld = dev_bf16(lay["lora_down"]) if lay["rank"] else None
    op, sc, lora = bq.svdq_w4a4_quantize_operand(dev_bf16(x_bits), dev_bf16(lay["smooth"]), ld, p)
    torch.cuda.synchronize()
    if p == "int4":
        got = op.cpu().numpy()
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{label}: {len(bad)} E4M3 code bytes differ, first {bad[:4].tolist()}: "
                               f"{[(hex(got[tuple(b)]), hex(want[tuple(b)])) for b in bad[:4]]}")
        got_sc = sc.cpu().numpy()
        assert got_sc.dtype == np.float32 and np.array_equal(got_sc.astype(np.float64), want_sc), \
            f"{label}: group scales differ"
    else:
        got = op.cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{label}: {len(bad)} operand values differ, first {bad[:4].tolist()}: "
                               f"{[(got[tuple(b)], want[tuple(b)]) for b in bad[:4]]}")
    if lay["rank"]:
        la = lora.cpu().numpy().astype(np.float64)
        err = np.abs(la - ref["lora_act"]).max()
        assert err <= 1e-4 * np.abs(ref["lora_act"]).max() + 1e-6, label
    print(f"[{label}] operand bit-exact ({got.size} values)", flush=True)


def check_k1(x_bits, lay, label):
    check_quantize_act(x_bits, lay, label)
    check_operand(x_bits, lay, label + " operand")


def act_layer(smooth_bits, rank, precision, rng):
    """The activation-side inputs of a layer (smooth, a random bf16 lora_down)."""
    K = len(smooth_bits)
    ld = S.to_bf16_bits(rng.standard_normal((rank, K)) * 0.05) if rank else np.zeros((0, K), np.uint16)
    return dict(precision=precision, smooth=smooth_bits, lora_down=ld, rank=rank)


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_quantize_act_config0(cfg0, precision):
    lay = prepared(cfg0["x"], cfg0["w"], cfg0["bias"], precision, 32)
    check_k1(cfg0["x"], lay, f"k1 cfg0 {precision}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("rank", [0, 16, 128])
def test_quantize_act_ragged(ragged, precision, rank):
    x, w, b = ragged
    lay = prepared(x, w, b, precision, rank, smooth="calibrated")
    check_k1(x, lay, f"k1 ragged {precision} r{rank}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("M,K,rank", [(33, 16384, 32), (70, 128, 16), (17, 16384, 128)])
def test_quantize_act_k_extremes(precision, M, K, rank):
    # codes and scales bit-exact at the largest and smallest K
    rng = np.random.default_rng(M + K + rank)
    x = S.activations(M, K, 3, rng)
    lay = prepared(x, S.weight(128, K, 0.02, rng), None, precision, rank, smooth="calibrated")
    check_k1(x, lay, f"k1 {precision} M={M} K={K} r{rank}")


@pytest.mark.parametrize("which", ["int4", "nvfp4"])
def test_quantize_act_full_size(cfg1_layers, which):
    c, lay4, layfp4 = cfg1_layers
    check_k1(c["x"], lay4 if which == "int4" else layfp4, f"k1 cfg1 {which}")


def test_quantize_act_edge_values():
    # zero rows, a denormal-only group, huge and tiny magnitudes, exact ties
    rng = np.random.default_rng(5)
    M, K = 40, 256
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[0] = 0
    xf[1, :64] = 1e-39
    xf[2] *= 1e30
    xf[3] *= 1e-30
    xf[4, :64] = np.arange(64) * 0.5
    xf[5, :16] = [6, 5, 3.5, 2.5, 1.75, 1.25, .75, .25, -6, -5, -3.5, -2.5, -1.75, -1.25, -.75, -.25]
    xf[6, :] = -0.0
    x = S.to_bf16_bits(xf)
    w = rng.standard_normal((64, K)) * 0.02
    for p in ("int4", "nvfp4"):
        lay = prepared(x, w, None, p, 16)
        check_k1(x, lay, f"k1 edge {p}")


@pytest.mark.parametrize("family", ["int4_codes", "nvfp4_scales", "nvfp4_codes"])
def test_quantize_act_rounding_ties(family):
    # exact rounding ties of the activation quantizer, through both the
    # packed-code export and the linear's own operand: int4 codes x / s =
    # n + 1/2; nvfp4 scales amax / 6 on every E4M3 midpoint (and the 448 /
    # 464 saturation edge); nvfp4 codes on every E2M1 midpoint.  (int4 group
    # scales have no bfloat16 ties: tests/test_tie_inputs.py.)
    x, sm, cases = {"int4_codes": T.int4_code_ties, "nvfp4_scales": T.nvfp4_scale_ties,
                    "nvfp4_codes": T.nvfp4_code_ties}[family]()
    p = family.split("_")[0]
    lay = act_layer(sm, 16, p, np.random.default_rng(len(cases)))
    check_k1(x, lay, f"k1 ties {family} ({len(cases)} groups)")


def scale_range_inputs():
    """int4 rows whose group scales span the bf16 range the quantizer makes:
    ordinary rows, scales far above 2^13 or below 2^-17, a row spread over
    2^-33 .. 2^-1, rows with one outlier group, zero rows, a row with one
    nonzero group (the product operand keeps every scale as fp32, so each
    class is exact)."""
    rng = np.random.default_rng(23)
    M, K = 100, 512
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[16:32] *= 3e5                      # scales far above 2^13
    xf[32:48] *= 1e-7                     # scales below 2^-17
    xf[48:64, 256:] *= 1e-9               # one row, scales 2^-33 .. 2^-1
    xf[64:80] = np.clip(xf[64:80], -3, 3)  # other groups: s ~ 0.4
    xf[64, 5] = 57088.0                   # s = bf16(57088 / 7) = 8160
    xf[65, 70] = 57344.0                  # s = 8192
    xf[66, 128:192] *= 1e-9
    xf[66, 130] = 7 * 2.0 ** -17          # smallest s = 2^-17
    xf[67, 128:192] *= 1e-9
    xf[67, 130] = 1.734375 * 2.0 ** -15   # smallest s just below 2^-17
    xf[80:84] = 0.0                       # zero rows
    xf[84, 64:] = 0.0                     # one nonzero group
    return S.to_bf16_bits(xf), rng


def test_quantize_operand_int4_scale_range():
    x, rng = scale_range_inputs()
    check_k1(x, act_layer(ones_smooth(x.shape[1]), 32, "int4", rng), "k1 int4 scale range")


# ------------------------------------------------------------------ kernel 2 partials
def check_partials(act_codes, w_codes, p, label):
    ref = L.svdq_partials_ref(act_codes, w_codes, p)
    got = bq.svdq_w4a4_gemm_partials(dev_u8(F.pack_nibbles(act_codes)), dev_u8(F.pack_nibbles(w_codes)), p)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.int64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{label}: {len(bad)} partials differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_partials_config0(cfg0, precision):
    lay = prepared(cfg0["x"], cfg0["w"], None, precision, 32)
    act = L.svdq_quantize_act(cfg0["x"], lay["smooth"], lay["lora_down"], precision)
    check_partials(act["codes"], lay["w_codes"], precision, f"partials cfg0 {precision}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_partials_all_codes(precision):
    # every nibble value on both sides (int4 includes the 0x8 "-0" code)
    rng = np.random.default_rng(7)
    a = rng.integers(0, 16, size=(200, 256)).astype(np.uint8)
    w = rng.integers(0, 16, size=(192, 256)).astype(np.uint8)
    check_partials(a, w, precision, f"partials random {precision}")


@pytest.mark.parametrize("which", ["int4", "nvfp4"])
def test_partials_full_size_sampled(cfg1_layers, which):
    c, lay4, layfp4 = cfg1_layers
    lay = lay4 if which == "int4" else layfp4
    act = L.svdq_quantize_act(c["x"][:130], lay["smooth"], lay["lora_down"], which)
    check_partials(act["codes"], lay["w_codes"][1024:1024 + 192], which, f"partials cfg1 {which}")


# ------------------------------------------------------------------ full linear
@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_linear_config0(cfg0, precision):
    lay = prepared(cfg0["x"], cfg0["w"], cfg0["bias"], precision, 32)
    y = run_linear(cfg0["x"], lay)
    assert_output(y, L.svdq_linear_ref(cfg0["x"], lay), f"linear cfg0 {precision}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("rank", [0, 16, 32, 128])
def test_linear_ragged(ragged, precision, rank):
    x, w, b = ragged
    lay = prepared(x, w, b, precision, rank, smooth="calibrated")
    y = run_linear(x, lay)
    assert_output(y, L.svdq_linear_ref(x, lay), f"linear ragged {precision} r{rank}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_linear_single_row_and_no_bias(ragged, precision):
    x, w, _ = ragged
    lay = prepared(x[:1], w, None, precision, 32, smooth="calibrated")
    y = run_linear(x[:1], lay)
    assert_output(y, L.svdq_linear_ref(x[:1], lay), f"linear M=1 {precision}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_linear_zero_identities(ragged, precision):
    x, w, b = ragged
    N, K = w.shape
    lay = prepared(x, np.zeros((N, K)), None, precision, 0)
    y = run_linear(x, lay)
    assert not host_bits(y).any() or not np.any(F.bf16_to_f32(host_bits(y)))
    lay = prepared(x, w, b, precision, 32, smooth="calibrated")
    y = run_linear(np.zeros_like(x), lay)
    assert np.array_equal(host_bits(y), np.broadcast_to(b, y.shape))


@pytest.mark.parametrize("which", ["int4", "nvfp4"])
def test_linear_full_size(cfg1_layers, which):
    c, lay4, layfp4 = cfg1_layers
    lay = lay4 if which == "int4" else layfp4
    y = run_linear(c["x"], lay)
    assert_output(y, L.svdq_linear_ref(c["x"], lay), f"linear cfg1 {which}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("M,K,N,rank", [(33, 16384, 320, 32), (70, 128, 64, 16), (5, 128, 448, 0),
                                        (300, 384, 320, 32)])
def test_linear_k_extremes(precision, M, K, N, rank):
    # K = 16384 (the largest accepted: 256 stages, not a multiple of the
    # loop's six), K = 128 (two stages) and K = 384 (an odd number of int4
    # stages, unsplit: the weight scales of two stages are loaded together);
    # N with a partial 192-column tile
    rng = np.random.default_rng(K + N + M)
    x = S.activations(M, K, 3, rng)
    lay = prepared(x, S.weight(N, K, 0.02, rng, spike_rank=2), S.bias(N, rng), precision, rank, smooth="calibrated")
    assert_output(run_linear(x, lay), L.svdq_linear_ref(x, lay), f"linear {precision} M={M} K={K} N={N} r{rank}")


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("M,K,N,rank", [(512, 3072, 3072, 32), (64, 640, 128, 16), (200, 1152, 576, 128),
                                        (256, 6144, 384, 32), (2048, 3072, 3072, 32), (64, 3200, 128, 16)])
def test_linear_split_k(precision, M, K, N, rank):
    # few output tiles: the product is split along K (int4 / nvfp4: 4 / 8
    # splits of 6 stages; 2 splits of 3 + 2 / of 5; 2 splits of 5 + 4 / 3 of
    # 6; 8 splits of 6 / 8 of 12; at 128 tiles 2 splits of 12 / 24; 5 splits
    # of 5 / 7 splits of 7 + 1) and the fp32 partials summed in order; the
    # low-rank term enters in split 0, the bias in the sum.  Odd stage counts
    # per split reach the loaders' last pair of stages, whose second stage
    # does not exist (the W scales of two stages share a load)
    rng = np.random.default_rng(M + K + N)
    x = S.activations(M, K, round(0.01 * K), rng)
    lay = prepared(x, S.weight(N, K, 0.02, rng, spike_rank=4), S.bias(N, rng), precision, rank, smooth="calibrated")
    y = run_linear(x, lay)
    rows = np.r_[0:24, M // 2:M // 2 + 8, M - 8:M] if M > 64 else np.arange(M)
    assert_output(y[rows], L.svdq_linear_ref(x[rows], lay), f"split-K {precision} M={M} K={K} N={N} r{rank}")


def test_linear_int4_scale_range():
    # int4 activations enter the product as fp8 codes with bf16 group scales
    # applied to each group's exact integer sum (the operand itself is checked
    # bit for bit in test_quantize_operand_int4_scale_range).  Rows of each
    # scale class, each class checked on its own.
    x, rng = scale_range_inputs()
    N, K = 192, x.shape[1]
    w = S.weight(N, K, 0.02, rng, spike_rank=4)
    b = S.bias(N, rng)
    lay = prepared(x, w, b, "int4", 32)
    y = run_linear(x, lay)
    yf = F.bf16_to_f32(host_bits(y)).astype(np.float64)
    ref = L.svdq_linear_ref(x, lay)
    assert np.all(np.isfinite(yf))
    classes = {"normal": list(range(0, 16)) + list(range(85, 100)), "huge": range(16, 32),
               "tiny": range(32, 48), "mixed": range(48, 64), "bounds": range(64, 80),
               "zero-ish": range(80, 85)}
    for name, rows in classes.items():
        rows = list(rows)
        for rr in rows if name == "bounds" else [rows]:
            sel = [rr] if name == "bounds" else rr
            _, excess, mre = L.output_errors(yf[sel], ref[sel])
            print(f"[int4 scale class {name} {sel if name == 'bounds' else ''}] excess {excess:.3e} MRE {mre:.3e}",
                  flush=True)
            assert excess <= 1e-2 and mre <= 2e-3, (name, sel)


def test_linear_deterministic_with_poisoned_workspace(ragged):
    x, w, b = ragged
    for p in ("int4", "nvfp4"):
        lay = prepared(x, w, b, p, 32, smooth="calibrated")
        y1 = host_bits(run_linear(x, lay, poison=0x00))
        y2 = host_bits(run_linear(x, lay, poison=0xFF))
        assert np.array_equal(y1, y2)


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_two_phase_entry_matches_linear(ragged, precision):
    # quantize + gemm as two calls reproduce the fused call bit for bit
    x, w, b = ragged
    lay = prepared(x, w, b, precision, 32, smooth="calibrated")
    layer = bq.SVDQLinear.from_numpy(lay)
    xd = dev_bf16(x)
    ws = torch.empty(layer.workspace_bytes(x.shape[0]), dtype=torch.uint8, device="cuda")
    bq.svdq_w4a4_quantize(xd, layer, ws)
    y2 = bq.svdq_w4a4_gemm(ws, x.shape[0], layer)
    y1 = layer(xd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y1), host_bits(y2))


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("M,K,rank", [(300, 512, 32), (37, 3072, 16), (4096, 3072, 32), (64, 384, 32),
                                      (70, 512, 48), (17, 16384, 32), (2048, 3072, 32), (5, 256, 0)])
def test_linear_kernel1_workspace(precision, M, K, rank):
    """Kernel 1 as the linear launches it (split along K for few rows: the
    low-rank slice partials added in order by a second kernel) against the
    operand export and the oracle: operand and group scales in the workspace
    bit for bit equal to the export's, lora_act within 1e-4 of the oracle's
    largest low-rank activation."""
    rng = np.random.default_rng(M + K + rank)
    x = S.activations(M, K, max(1, K // 100), rng)
    lay = act_layer(L.smooth_factors(x, S.weight(64, K, 0.02, rng, spike_rank=0)), rank, precision, rng)
    ref = L.svdq_quantize_act(x, lay["smooth"], lay["lora_down"], precision)
    xd, smd = dev_bf16(x), dev_bf16(lay["smooth"])
    ldd = dev_bf16(lay["lora_down"]) if rank else None
    op, sc, _ = bq.svdq_w4a4_quantize_operand(xd, smd, ldd, precision)
    G = 64 if precision == "int4" else 16
    layer = bq.SVDQLinear(torch.zeros((64, K // 2), dtype=torch.uint8, device="cuda"),
                          torch.zeros((64, K // G), dtype=torch.bfloat16 if precision == "int4" else torch.uint8,
                                      device="cuda"),
                          smd, ldd, torch.zeros((64, rank), dtype=torch.bfloat16, device="cuda") if rank else None,
                          None, precision, wtscale=1.0)
    ws = torch.empty(layer.workspace_bytes(M), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    bq.svdq_w4a4_quantize(xd, layer, ws)
    torch.cuda.synchronize()
    rnd = lambda v: (v + 255) // 256 * 256
    w = ws.cpu().numpy()
    opb = M * K * (1 if precision == "int4" else 2)
    assert np.array_equal(w[:opb], op.cpu().numpy().view(np.uint8).reshape(-1)), "operand differs from the export"
    off = rnd(opb)
    if precision == "int4":
        # the workspace holds the bf16 bits of the export's fp32 scales (bf16 values)
        scb = M * (K // 64) * 2
        sc32 = sc.cpu().numpy().view(np.uint32).reshape(-1)
        assert np.all(sc32 & 0xFFFF == 0), "export scales are not bf16 values"
        assert np.array_equal(w[off:off + scb].view(np.uint16), (sc32 >> 16).astype(np.uint16)), "group scales differ"
        off += rnd(scb)
    if rank:
        la = w[off:off + M * rank * 4].view(np.float32).reshape(M, rank).astype(np.float64)
        err = np.abs(la - ref["lora_act"]).max()
        tol = 1e-4 * np.abs(ref["lora_act"]).max() + 1e-6
        print(f"[kernel 1 workspace {precision} M={M} K={K} r{rank}] lora_act max err {err:.3e} (tol {tol:.3e})",
              flush=True)
        assert err <= tol


# ------------------------------------------------------------------ AWQ
def run_awq(x_bits, lay):
    layer = bq.AWQLinear.from_numpy(lay)
    y = layer(dev_bf16(x_bits))
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M", [1, 2, 16, 33])
def test_awq_ragged(M):
    rng = np.random.default_rng(M)
    K, N = 384, 320
    w = rng.standard_normal((N, K)) * 0.02
    lay = L.prepare_awq_layer(w, S.bias(N, rng))
    x = S.activations(M, K, 0, rng)
    assert_output(run_awq(x, lay), L.awq_linear_ref(x, lay), f"awq ragged M={M}")


@pytest.mark.parametrize("M,K,N", [(1, 128, 64), (3, 640, 128), (4, 1152, 192), (5, 8192, 64),
                                   (2, 16384, 64), (17, 3200, 128), (1, 1024, 64), (1, 2048, 192),
                                   (1, 4096, 320), (1, 8192, 64), (2, 2048, 192), (2, 4096, 320)])
def test_awq_shapes(M, K, N):
    # X-row tiles of 1, 2, 4 and 16 rows; K from one group pair to the maximum
    # (a scale table wider than one load batch); partial 4-group steps; the
    # the one-token VALU path for K = 1024 .. 4096 (and K = 8192 past it);
    # two tokens at the same K on the matrix-instruction kernel
    rng = np.random.default_rng(K + M)
    w = rng.standard_normal((N, K)) * 0.02
    lay = L.prepare_awq_layer(w, S.bias(N, rng))
    x = S.activations(M, K, 0, rng)
    assert_output(run_awq(x, lay), L.awq_linear_ref(x, lay), f"awq M={M} K={K} N={N}")


# ------------------------------------------------------------------ MLP pair and stack shapes
# Full-size layers, checked on a sample of rows (first, middle and last tiles,
# ragged positions) against the oracle on the same input.
SAMPLE_ROWS = np.r_[0:40, 255:258, 2047:2060, 4090:4096]


@pytest.fixture(scope="module")
def mlp_up():
    c = S.config2()
    x = c["proj"]["x"]
    lay = prepared(x, c["w_up"], c["b_up"], "nvfp4", 32, smooth="calibrated")
    h = run_linear(x, lay)
    return c, x, lay, h


def test_mlp_pair_up_config2_sampled(mlp_up):
    # nvfp4 MLP up-projection 3072 -> 12288 at M = 4096
    _, x, lay, h = mlp_up
    assert_output(h[SAMPLE_ROWS], L.svdq_linear_ref(x[SAMPLE_ROWS], lay), "mlp up 3072->12288")


def test_mlp_pair_down_config2_sampled(mlp_up):
    # down-projection 12288 -> 3072 at M = 4096 on post-GELU activations: the
    # oracle's bf16 GELU of synthetic activations with outlier channels
    c = mlp_up[0]
    g = L.gelu_bf16(S.activations(4096, 12288, 123, np.random.default_rng(12288)))
    lay = prepared(g, c["w_down"], c["b_down"], "nvfp4", 32, smooth="calibrated")
    y = run_linear(g, lay)
    assert_output(y[SAMPLE_ROWS], L.svdq_linear_ref(g[SAMPLE_ROWS], lay), "mlp down 12288->3072")


# The fused MLP never exposes its up output h; its parity tests use up layers
# on which the fp32 product is exact (tests/exact_mlp.py), so that bf16(h) is
# unique and the oracle computes the whole chain from x alone.  The fused
# kernel's main loop is the plain linear's, checked on general inputs above.
def fused_mlp_ref(x, lay_up, w_down, b_down, rank_down):
    h = F.bf16_bits_f64(L.svdq_linear_ref(x, lay_up))
    lay_down = prepared(L.gelu_bf16(h), w_down, b_down, "nvfp4", rank_down, smooth="calibrated")
    return lay_down, L.mlp_gelu_ref(h, lay_down)


def test_mlp_gelu_fused_config2_sampled(mlp_up):
    # the fused MLP (GELU and the nvfp4 quantization for the down projection
    # in the up projection's epilogue) at 3072 -> 12288 -> 3072, M = 4096,
    # rank 32 in both layers
    c = mlp_up[0]
    x, lay_up = exact_up_problem(4096, 3072, 12288, "nvfp4", 32, np.random.default_rng(77))
    lay_down, y_ref = fused_mlp_ref(x[SAMPLE_ROWS], lay_up, c["w_down"], c["b_down"], 32)
    y = bq.svdq_w4a4_mlp_gelu(dev_bf16(x), bq.SVDQLinear.from_numpy(lay_up), bq.SVDQLinear.from_numpy(lay_down))
    torch.cuda.synchronize()
    assert_output(y[SAMPLE_ROWS], y_ref, "fused mlp 3072->12288->3072")


# rows of the first, middle and last 256-row tiles for the chain check below
CHAIN_ROWS = np.r_[0:8, 255:258, 2047:2053, 4090:4096]


def ambiguous_h(x_rows, lay_up):
    """The oracle's up output h (fp64) for x_rows, its bf16 rounding, and the
    elements whose bf16 rounding is not decided within the radius
    delta = 2^-16 (|h| + sum_j |lora_act_j up_j|): the GPU's h differs from
    the fp64 one by its fp32 accumulation and, mostly, by its bf16 hi + lo
    evaluation of the low-rank branch, whose error scales with the branch's
    terms.  On config 2's up layer every h the GPU rounds the other way lies
    within 3.5e-6 of that scale from its midpoint, so the radius (1.5e-5) has
    a margin of 4; it stays far below a bf16 spacing (2^-8 relative).
    Returns (h64, hb, lo, hi, amb): lo / hi the bf16 roundings of h -+ delta."""
    p = lay_up["precision"]
    act = L.svdq_quantize_act(x_rows, lay_up["smooth"], lay_up["lora_down"], p)
    h64 = L.svdq_linear_ref(x_rows, lay_up, act=act)
    lora_abs = np.abs(act["lora_act"]) @ np.abs(F.bf16_to_f32(lay_up["lora_up"]).astype(np.float64)).T
    delta = 2.0 ** -16 * (np.abs(h64) + lora_abs)
    hb, lo, hi = F.bf16_bits_f64(h64), F.bf16_bits_f64(h64 - delta), F.bf16_bits_f64(h64 + delta)
    return h64, hb, lo, hi, (lo != hb) | (hi != hb)


def chain_allowance(hb, lo, hi, amb, lay_down, max_amb=12):
    """Per output element of the down layer, the largest change a different
    valid rounding of h can make: for each 16-column group of the down
    layer's input holding ambiguous elements, every choice of their roundings
    (lo or hi) goes through the oracle's GELU, smoothing and nvfp4 quantizer,
    and the largest |change| of the group's contribution (4-bit product and
    low-rank branch) over the choices is added up over the groups."""
    import itertools
    from scipy import sparse
    R, H = hb.shape
    wd = L.dequant(lay_down["w_codes"], lay_down["wscales"], "nvfp4") * float(lay_down["wtscale"])
    ld = F.bf16_to_f32(lay_down["lora_down"]).astype(np.float64)
    lu = F.bf16_to_f32(lay_down["lora_up"]).astype(np.float64)
    sm = lay_down["smooth"]
    allow = np.zeros((R, wd.shape[0]))
    ngroups = 0
    for m in range(R):
        gids = np.unique(np.flatnonzero(amb[m]) // 16)
        if not len(gids):
            continue
        ngroups += len(gids)
        rows_h, owner = [], []           # every choice of every ambiguous group, as 16 h values
        for gi, g in enumerate(gids):
            cols = np.arange(16 * g, 16 * g + 16)
            idx = np.flatnonzero(amb[m, cols])
            assert len(idx) <= max_amb, "too many ambiguous values in one group"
            for choice in itertools.product(*[(lo[m, cols[i]], hi[m, cols[i]]) for i in idx]):
                hh = hb[m, cols].copy()
                hh[idx] = choice
                rows_h.append(hh)
                owner.append(gi)
        owner = np.array(owner)
        cols_all = (16 * gids[owner])[:, None] + np.arange(16)[None, :]
        base = hb[m, cols_all]

        def quant(hbits):
            xh = L.smoothed_activations(L.gelu_bf16(hbits).reshape(1, -1), sm[cols_all].reshape(-1))
            xh = xh.reshape(hbits.shape)
            codes, sc = Q.quantize_nvfp4_act(xh, 16)
            return L.dequant(codes, sc, "nvfp4"), xh.astype(np.float64)
        d1, x1 = quant(np.array(rows_h))
        d0, x0 = quant(base)
        C = len(owner)
        rr = np.repeat(np.arange(C), 16)
        dD = sparse.csr_matrix(((d1 - d0).ravel(), (rr, cols_all.ravel())), shape=(C, H))
        dX = sparse.csr_matrix(((x1 - x0).ravel(), (rr, cols_all.ravel())), shape=(C, H))
        change = np.abs(dD @ wd.T + (dX @ ld.T) @ lu.T)          # [choices, N]
        starts = np.flatnonzero(np.r_[True, owner[1:] != owner[:-1]])
        allow[m] = np.maximum.reduceat(change, starts, axis=0).sum(axis=0)
    return allow, ngroups


def test_mlp_gelu_fused_config2_own_weights_sampled(mlp_up):
    # The fused MLP on config 2's own prepared up layer (calibrated smoothing,
    # SVD split, nvfp4 residual).  Its bf16 h is not unique: where the fp64 h
    # lies within the GPU's accuracy of a bf16 midpoint either rounding is
    # correct, and one flipped h can move the E4M3 scale of its group in the
    # down layer's quantization (measured: 0.3 % of h values flip, and the
    # unfused chain of GPU linears shows the same output change as the fused
    # one).  So: (1) every element where the GPU's up output rounds h
    # differently from the oracle is one the oracle marks ambiguous; (2) each
    # output meets the bar up to the largest change that any choice of the
    # ambiguous roundings can make (chain_allowance); MRE as usual.
    c, x, lay_up, h_plain = mlp_up
    rows = CHAIN_ROWS
    xs = x[rows]
    h64, hb, lo, hi, amb = ambiguous_h(xs, lay_up)
    flips = host_bits(h_plain)[rows] != hb
    print(f"[fused mlp own weights] ambiguous h: {int(amb.sum())}, GPU flips: {int(flips.sum())} "
          f"of {hb.size}", flush=True)
    assert not np.any(flips & ~amb), "the GPU's h rounds differently outside the ambiguous set"
    lay_down = prepared(L.gelu_bf16(hb), c["w_down"], c["b_down"], "nvfp4", 32, smooth="calibrated")
    y_ref = L.mlp_gelu_ref(hb, lay_down)
    allow, groups = chain_allowance(hb, lo, hi, amb, lay_down)
    y = bq.svdq_w4a4_mlp_gelu(dev_bf16(x), bq.SVDQLinear.from_numpy(lay_up), bq.SVDQLinear.from_numpy(lay_down))
    torch.cuda.synchronize()
    yf = F.bf16_to_f32(host_bits(y)[rows]).astype(np.float64)
    assert np.all(np.isfinite(yf))
    err = np.abs(yf - y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2))
    excess = np.max(err - L.bf16_half_ulp(y_ref) - allow) / rms
    mre = err.sum() / np.abs(y_ref).sum()
    print(f"[fused mlp own weights] {groups} ambiguous groups; max allowance/RMS {allow.max() / rms:.3e}; "
          f"max|err|/RMS {err.max() / rms:.3e}; beyond half-ulp + allowance {excess:.3e}; MRE {mre:.3e}", flush=True)
    assert excess <= 1e-2 and mre <= 2e-3


@pytest.mark.parametrize("M,up_prec,ranks", [(1, "nvfp4", (32, 32)), (37, "int4", (32, 32)),
                                             (300, "nvfp4", (0, 16)), (300, "int4", (16, 0)),
                                             (257, "nvfp4", (128, 128))])
def test_mlp_gelu_fused_ragged(M, up_prec, ranks):
    # H = 640: the last 192-column tile of the up projection is partial; M
    # ragged against the 256-row tiles; every rank block path of the epilogue
    rng = np.random.default_rng(M + ranks[0])
    K, H, N = 256, 640, 320
    x, lay_up = exact_up_problem(M, K, H, up_prec, ranks[0], rng)
    lay_down, y_ref = fused_mlp_ref(x, lay_up, S.weight(N, H, 0.02, rng), S.bias(N, rng), ranks[1])
    y = bq.svdq_w4a4_mlp_gelu(dev_bf16(x), bq.SVDQLinear.from_numpy(lay_up), bq.SVDQLinear.from_numpy(lay_down))
    torch.cuda.synchronize()
    assert_output(y, y_ref, f"fused mlp M={M} {up_prec} r{ranks}")


def test_mlp_gelu_deterministic():
    # the down layer's low-rank activations are summed per column tile and
    # the tiles added in order: the same inputs give the same bits, whatever
    # the workspace held before
    rng = np.random.default_rng(2)
    x, lay_up = exact_up_problem(300, 256, 640, "nvfp4", 32, rng)
    lay_down, _ = fused_mlp_ref(x[:4], lay_up, S.weight(320, 640, 0.02, rng), S.bias(320, rng), 32)
    up, down = bq.SVDQLinear.from_numpy(lay_up), bq.SVDQLinear.from_numpy(lay_down)
    xd = dev_bf16(x)
    need = bq.mlp_workspace_bytes(300, up, down)
    outs = []
    for poison in (0x00, 0xFF, 0x7F):
        ws = torch.full((need,), poison, dtype=torch.uint8, device="cuda")
        outs.append(host_bits(bq.svdq_w4a4_mlp_gelu(xd, up, down, workspace=ws)))
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


def test_mlp_gelu_rejects_int4_down():
    rng = np.random.default_rng(5)
    x = S.activations(64, 256, 0, rng)
    up = bq.SVDQLinear.from_numpy(prepared(x, S.weight(256, 256, 0.02, rng), None, "nvfp4", 16))
    down = bq.SVDQLinear.from_numpy(prepared(x, S.weight(128, 256, 0.02, rng), None, "int4", 16))
    with pytest.raises(bq.SvdqError) as e:
        bq.svdq_w4a4_mlp_gelu(dev_bf16(x), up, down)
    assert e.value.status == -2


def test_stack_qkv_sampled():
    # the DiT stack's fused QKV shape, 3072 -> 9216 nvfp4 rank 32 at 4096 tokens
    x, w, b = S.svdq_problem(4096, 3072, 9216, seed=5, n_outliers=31)
    lay = prepared(x, w, b, "nvfp4", 32, smooth="calibrated")
    y = run_linear(x, lay)
    assert_output(y[SAMPLE_ROWS], L.svdq_linear_ref(x[SAMPLE_ROWS], lay), "stack qkv 3072->9216")


def test_awq_config3():
    c = S.config3()
    lay = L.prepare_awq_layer(c["w"], c["bias"])
    for M, x in c["xs"].items():
        assert_output(run_awq(x, lay), L.awq_linear_ref(x, lay), f"awq cfg3 M={M}")


def test_awq_no_bias_and_extreme_codes():
    rng = np.random.default_rng(3)
    K, N = 256, 128
    w = rng.standard_normal((N, K)) * 0.02
    w[0] = 0.0           # all-zero rows -> zero scale groups
    w[1, :64] = 5.0      # one-sided range (min clamps to 0)
    lay = L.prepare_awq_layer(w, None)
    x = S.activations(4, K, 0, rng)
    assert_output(run_awq(x, lay), L.awq_linear_ref(x, lay), "awq extremes")


# ------------------------------------------------------------------ QKV + RMSNorm + RoPE
def bf16_ulp(v):
    return 2.0 * L.bf16_half_ulp(v)


def check_qkv(x, lay, heads, qn, kn, cos, sin, eps, label, rows=None):
    """The fused QKV call against the oracle.  v: bit for bit the plain
    linear's output where that is not split along K, and the output bar
    (max |err| - half-ulp <= 1e-2 RMS, MRE <= 2e-3).  q | k pass through two bf16 roundings
    (n = bf16(RMSNorm(h)), then the rotation's); the GPU's fp32 chain and the
    oracle's fp64 one can round n differently, and h itself can differ in its
    last place, so each output may also differ by two ulps of each n it
    combines: |err| <= half-ulp(out) + 2 (ulp(n_a) |c| + ulp(n_b) |s|) +
    1e-2 RMS, with MRE <= 2e-3."""
    D = len(qn)
    layer = bq.SVDQLinear.from_numpy(lay)
    xd = dev_bf16(x)
    y = bq.svdq_w4a4_qkv_rmsnorm_rope(xd, layer, heads, dev_bf16(qn), dev_bf16(kn),
                                      torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), eps)
    plain = layer(xd)
    torch.cuda.synchronize()
    rows = np.arange(x.shape[0]) if rows is None else rows
    ref = L.qkv_norm_rope_ref(x[rows], lay, heads, qn, kn, eps, cos[rows], sin[rows])
    qk = 2 * heads * D
    yb = host_bits(y)[rows]
    if ksplit(x.shape[0], 3 * heads * D, x.shape[1], lay["precision"]) == 1:
        # the plain linear sums in the same order
        assert np.array_equal(yb[:, qk:], host_bits(plain)[rows][:, qk:]), label
    assert_output(torch.from_numpy(yb[:, qk:].view(np.int16).copy()).view(torch.bfloat16), ref[:, qk:], label + " v")
    # q | k with the allowance for the intermediate rounding
    R = len(rows)
    h = F.bf16_bits_f64(L.svdq_linear_ref(x[rows], lay))[:, :qk].reshape(R, 2, heads, D)
    n = np.stack([F.bf16_to_f32(L.rmsnorm_bf16(h[:, p], w, eps)).astype(np.float64) for p, w in ((0, qn), (1, kn))],
                 axis=1)
    c, s_ = np.abs(cos[rows])[:, None, None, :], np.abs(sin[rows])[:, None, None, :]
    ua, ub = bf16_ulp(n[..., 0::2]), bf16_ulp(n[..., 1::2])
    allow = np.empty_like(n)
    allow[..., 0::2] = 2 * (ua * c + ub * s_)
    allow[..., 1::2] = 2 * (ua * s_ + ub * c)
    allow = allow.reshape(R, qk)
    got = F.bf16_to_f32(yb[:, :qk]).astype(np.float64)
    want = ref[:, :qk]
    err = np.abs(got - want)
    rms = np.sqrt(np.mean(want ** 2))
    excess = np.max(err - L.bf16_half_ulp(want) - allow) / rms
    mre = err.sum() / np.abs(want).sum()
    print(f"[{label} q|k] max|err|/RMS={err.max() / rms:.3e} (beyond the allowance {excess:.3e}) MRE={mre:.3e} "
          f"elements beyond half-ulp + 1e-2 RMS: {int(np.sum(err - L.bf16_half_ulp(want) > 1e-2 * rms))}", flush=True)
    assert np.all(np.isfinite(got))
    assert excess <= 1e-2 and mre <= 2e-3, label


@pytest.mark.parametrize("M,heads,D,precision,rank", [
    (1, 1, 128, "nvfp4", 32), (37, 2, 128, "int4", 16), (300, 3, 128, "nvfp4", 0), (257, 2, 128, "int4", 32),
    (300, 1, 128, "nvfp4", 128),
    # head dims 64 (two heads per column tile, one of them split between the
    # tile's two waves) and 32 (four per tile), heads of q and k in one tile
    (1, 1, 64, "int4", 32), (37, 3, 64, "nvfp4", 16), (300, 5, 64, "int4", 0), (257, 2, 32, "nvfp4", 32),
    (300, 6, 32, "int4", 128), (64, 10, 32, "nvfp4", 16)])
def test_qkv_rmsnorm_rope_ragged(M, heads, D, precision, rank):
    # M ragged against the 256-row tiles; heads D / 64 column tiles per call
    rng = np.random.default_rng(M * 7 + heads + D)
    K, N = 256, 3 * heads * D
    x = S.activations(M, K, 3, rng)
    lay = prepared(x, S.weight(N, K, 0.05, rng, spike_rank=2), S.bias(N, rng), precision, rank, smooth="calibrated")
    qn, kn = S.norm_weight(D, rng), S.norm_weight(D, rng)
    cos, sin = S.rope_tables(M, D, offset=M)
    check_qkv(x, lay, heads, qn, kn, cos, sin, 1e-6, f"qkv M={M} H={heads} D={D} {precision} r{rank}")


def test_qkv_rmsnorm_rope_dit_sampled():
    # the DiT attention projection: 4096 tokens, 24 heads of 128 (3072 -> 9216), nvfp4 rank 32
    x, w, b = S.svdq_problem(4096, 3072, 9216, seed=5, n_outliers=31)
    lay = prepared(x, w, b, "nvfp4", 32, smooth="calibrated")
    rng = np.random.default_rng(24)
    qn, kn = S.norm_weight(128, rng), S.norm_weight(128, rng)
    cos, sin = S.rope_tables(4096, 128)
    check_qkv(x, lay, 24, qn, kn, cos, sin, 1e-6, "qkv dit 3072->9216", rows=SAMPLE_ROWS)


def test_qkv_rejects_head_dim():
    # head dim 256: a q or k head would span two column tiles
    rng = np.random.default_rng(1)
    x = S.activations(8, 256, 0, rng)
    lay = bq.SVDQLinear.from_numpy(prepared(x, S.weight(768, 256, 0.05, rng), None, "nvfp4", 16))
    cos, sin = (torch.from_numpy(t).cuda() for t in S.rope_tables(8, 256))
    q = dev_bf16(S.norm_weight(256, rng))
    with pytest.raises(bq.SvdqError) as e:
        bq.svdq_w4a4_qkv_rmsnorm_rope(dev_bf16(x), lay, 1, q, q, cos, sin)
    assert e.value.status == -2
