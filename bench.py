#!/usr/bin/env python3
"""Benchmark of the gfx950 SVDQ W4A4 linear; prints ONE JSON line.

Workload (the headline): one svdq_w4a4 int4 linear of DiT attention-projection
shape, X bf16 [4096, 3072] (1 % outlier channels), W [3072, 3072], rank 32,
group 64 -- a "step" is one svdq_w4a4_linear call (kernel 1 + kernel 2), inputs
resident in HBM.  value = effective TOPS = 2 M N K / step time.

Also measured in the same run (reported under "extra"):
  * the nvfp4 variant of the same layer;
  * the same int4 layer on one GPU's share of the tokens when 8 GPUs split
    them (M = 512);
  * per-kernel durations (HIP events on the launch stream) of
    quantize_act_lora_down and gemm_w4a4_lora_up, from which the roofline
    object of the dominant kernel (gemm_w4a4_lora_up) is computed;
  * awq_w4a16 at M in {1, 2, 16}, K=3072, N=18432, rotating over 12 weight
    copies (382 MB > the 256 MB last-level cache) so weights come from HBM,
    timed as a captured graph of 48 launches replayed (a ~10 us kernel is
    close to the host's per-call launch cost, which the graph leaves out);
  * the nvfp4 MLP pair 3072 -> 12288 -> 3072 at M=4096 (exact-erf GELU on the
    bf16 up output, a torch op, between the two library calls), and the same
    pair fused (svdq_w4a4_mlp_gelu: GELU and the down projection's
    quantization in the up projection's epilogue);
  * the attention QKV projection 3072 -> 9216 (24 heads of 128, nvfp4) with
    per-head RMSNorm and RoPE on q and k, as the linear plus torch ops and
    fused (svdq_w4a4_qkv_rmsnorm_rope);
  * offline weight preparation of a 9216 x 3072 nvfp4 layer on the GPU;
  * the DiT stack per pass: 24 blocks of QKV 3072->9216, out 3072->3072, MLP
    up/GELU/down (svdq nvfp4, rank 32, 4096 tokens) and the adaLN modulation
    linear 3072->18432 (awq_w4a16, one token; its 24 launches per pass are
    timed from a replayed graph), 8 passes (--no-stack skips it); also with
    the per-head RMSNorm and RoPE of q and k as torch ops, and with the QKV
    and MLP fusions.
The headline int4 and nvfp4 legs run on the config-1 layer itself, prepared on
the GPU by this library (smoothing calibrated on X, rank-32 split, residual
packing) from the synthetic config-1 weight; the other legs use random but
valid packed layers of their shapes (values do not change the work they do).
Parity with the oracle is the job of tests/.  Before the counted warm-up steps
every timed leg runs for a fixed wall time (--warm-seconds) so that the GPU
clock has settled whatever --warmup is.  The cpu_baseline leg times the CPU
oracle on bounded samples of configs 1-4 (config 4 extrapolated from one
block's layers).
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective W4A4 linear TOPS at M=4096,K=N=3072 (int4 & nvfp4); % MFMA/HBM roofline"
PEAK = {"fp8": 5000.0, "f16": 2500.0, "bf16": 2500.0, "hbm": 8000.0}  # TFLOP/s, GB/s (MI355X dense)
KERNEL_SOURCES = {"gemm_w4a4_lora_up": ["gemm_w4a4.hip", "device_common.hpp"],
                  "quantize_act_lora_down": ["quantize_act.hip", "device_common.hpp"],
                  "awq_w4a16": ["awq_gemv.hip", "device_common.hpp"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "bit_quantized_linear_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}|{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def bench_mlp_pair(bq, S, torch, np, x, M, K, rank, stream, hidden=12288, reps=50):
    """The nvfp4 MLP pair at M tokens: up K -> hidden, exact-erf GELU on the bf16
    output (a torch op between the two library calls), down hidden -> K."""
    import torch.nn.functional as Fn
    log("timing the nvfp4 MLP pair ...")
    r_up, r_dn = S.streams(11, 2)
    up = bq.SVDQLinear.from_numpy(S.random_svdq_layer(hidden, K, "nvfp4", rank, r_up))
    down = bq.SVDQLinear.from_numpy(S.random_svdq_layer(K, hidden, "nvfp4", rank, r_dn))
    ws_up = torch.empty(up.workspace_bytes(M), dtype=torch.uint8, device="cuda")
    ws_dn = torch.empty(down.workspace_bytes(M), dtype=torch.uint8, device="cuda")
    h = torch.empty((M, hidden), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    g = [Fn.gelu(h)]
    f_up = lambda: up(x, out=h, workspace=ws_up)
    f_gelu = lambda: g.__setitem__(0, Fn.gelu(h))
    f_dn = lambda: down(g[0], out=y, workspace=ws_dn)

    def pair():
        f_up()
        f_gelu()
        f_dn()
    # the fused MLP: GELU and the down projection's quantization in the up
    # projection's epilogue (no [M, hidden] bf16 tensor)
    ws_mlp = torch.empty(bq.mlp_workspace_bytes(M, up, down), dtype=torch.uint8, device="cuda")
    y_f = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    f_fused = lambda: bq.svdq_w4a4_mlp_gelu(x, up, down, out=y_f, workspace=ws_mlp)
    for _ in range(10):
        pair()
        f_fused()
    t_up, t_gelu, t_dn = (time_events(f, reps, stream) for f in (f_up, f_gelu, f_dn))
    t_pair = time_events(pair, reps, stream)
    t_fused = time_events(f_fused, reps, stream)
    ops = 2.0 * M * hidden * K * 2
    return {"up_us": round(t_up * 1e3, 2), "gelu_us": round(t_gelu * 1e3, 2), "down_us": round(t_dn * 1e3, 2),
            "pair_us": round(t_pair * 1e3, 2),
            "svdq_TOPS": round(ops / ((t_up + t_dn) * 1e-3) / 1e12, 1),
            "pair_TOPS_incl_gelu": round(ops / (t_pair * 1e-3) / 1e12, 1),
            "fused_pair_us": round(t_fused * 1e3, 2),
            "fused_pair_TOPS": round(ops / (t_fused * 1e-3) / 1e12, 1),
            "fused_speedup": round(t_pair / t_fused, 3)}


def torch_norm_rope(y, heads, qn, kn, cos, sin, eps=1e-6):
    """The unfused form of the QKV epilogue as separate torch ops on the bf16
    projection (per-head RMSNorm in fp32 with a bf16 weight, then RoPE on
    interleaved pairs in fp32), as a bf16 DiT attention block runs them."""
    import torch
    M = y.shape[0]
    q, k, v = y.view(M, 3, heads, 128).unbind(1)

    def norm(t, w):
        tf = t.float()
        tf = tf * torch.rsqrt(tf.pow(2).mean(-1, keepdim=True) + eps)
        return tf.to(torch.bfloat16) * w

    def rope(t):
        tf = t.float().view(M, heads, 64, 2)
        a, b = tf[..., 0], tf[..., 1]
        c, s = cos[:, None, :], sin[:, None, :]
        return torch.stack((a * c - b * s, a * s + b * c), -1).view(M, heads, 128).to(torch.bfloat16)
    return rope(norm(q, qn)), rope(norm(k, kn)), v


def bench_qkv(bq, S, torch, np, M, K, rank, stream, heads=24, reps=50):
    """The DiT attention projection 3072 -> 9216 (24 heads of 128, nvfp4, rank
    32) with per-head RMSNorm and RoPE on q and k: the linear followed by the
    torch ops, against svdq_w4a4_qkv_rmsnorm_rope (the same in the linear's
    epilogue)."""
    log("timing the fused QKV projection ...")
    N = 3 * heads * 128
    rl, rx, rn = S.streams(17, 3)
    layer = bq.SVDQLinear.from_numpy(S.random_svdq_layer(N, K, "nvfp4", rank, rl))
    x = torch.from_numpy(S.activations(M, K, round(0.01 * K), rx).view(np.int16).copy()).view(torch.bfloat16).cuda()
    qn, kn = (torch.from_numpy(S.norm_weight(128, rn).view(np.int16).copy()).view(torch.bfloat16).cuda()
              for _ in range(2))
    cos, sin = (torch.from_numpy(t).cuda() for t in S.rope_tables(M, 128))
    ws = torch.empty(layer.workspace_bytes(M), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yf = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    keep = [None]
    f_lin = lambda: layer(x, out=y, workspace=ws)
    f_ops = lambda: keep.__setitem__(0, torch_norm_rope(y, heads, qn, kn, cos, sin))
    f_unfused = lambda: (f_lin(), f_ops())
    f_fused = lambda: bq.svdq_w4a4_qkv_rmsnorm_rope(x, layer, heads, qn, kn, cos, sin, out=yf, workspace=ws)
    for _ in range(10):
        f_unfused()
        f_fused()
    t_lin, t_ops, t_unf, t_fus = (time_events(f, reps, stream) for f in (f_lin, f_ops, f_unfused, f_fused))
    ops = 2.0 * M * N * K
    return {"linear_us": round(t_lin * 1e3, 2), "torch_norm_rope_us": round(t_ops * 1e3, 2),
            "unfused_us": round(t_unf * 1e3, 2), "fused_us": round(t_fus * 1e3, 2),
            "fused_TOPS": round(ops / (t_fus * 1e-3) / 1e12, 1),
            "epilogue_cost_us": round((t_fus - t_lin) * 1e3, 2), "fused_speedup": round(t_unf / t_fus, 3)}


def bench_weight_prep(bq, S, torch, np, stream, N=9216, K=3072, M=4096, rank=32, reps=20):
    """Offline preparation of the QKV-shaped nvfp4 layer on the GPU: the
    smoothing factors and the residual packing (this library's kernels), and
    the whole prepare_layer call (with torch's randomized SVD)."""
    import time as _t
    log("timing the GPU weight preparation ...")
    rx, rw = S.streams(19, 2)
    x = torch.from_numpy(S.activations(M, K, round(0.01 * K), rx).view(np.int16).copy()).view(torch.bfloat16).cuda()
    w = torch.from_numpy(S.weight(N, K, 0.02, rw, spike_rank=8).astype(np.float32)).cuda()
    ws = torch.empty(bq.lib().svdq_w4a4_prep_workspace_bytes(K), dtype=torch.uint8, device="cuda")
    t_smooth = time_events(lambda: bq.smooth_factors(x, w, workspace=ws), reps, stream)
    t_pack = time_events(lambda: bq.pack_weight(w, "nvfp4", workspace=ws), reps, stream)
    bq.prepare_layer(w, x, rank, "nvfp4")
    torch.cuda.synchronize()
    t0 = _t.perf_counter()
    for _ in range(3):
        bq.prepare_layer(w, x, rank, "nvfp4")
    torch.cuda.synchronize()
    t_prep = (_t.perf_counter() - t0) / 3
    return {"shape": f"{N}x{K} nvfp4 rank {rank}, {M} calibration tokens",
            "smooth_factors_us": round(t_smooth * 1e3, 2), "pack_weight_us": round(t_pack * 1e3, 2),
            "prepare_layer_ms": round(t_prep * 1e3, 2)}


def bench_stack(bq, S, torch, np, M, rank, stream):
    """DiT stack per pass: every block runs QKV, out, MLP up, GELU, MLP down (svdq
    nvfp4, rank 32, M tokens, each linear on its own pre-generated activation,
    down on GELU(up)) and the adaLN modulation linear (awq_w4a16, one token).
    Each layer shape is generated once and copied into one device buffer per
    block."""
    import torch.nn.functional as Fn
    log("timing the DiT stack ...")
    blocks, passes = S.STACK["blocks"], S.STACK["passes"]
    shapes = S.STACK_LAYERS
    rs = S.streams(13, len(shapes) + 6)
    layers = {}
    for i, (name, Kl, Nl) in enumerate(shapes):
        base = S.random_svdq_layer(Nl, Kl, "nvfp4", rank, rs[i])
        layers[name] = [bq.SVDQLinear.from_numpy(base) for _ in range(blocks)]
    Ka, Na = S.STACK["adaln"]
    ada_base = S.random_awq_layer(Na, Ka, rs[len(shapes)])
    ada = [bq.AWQLinear.from_numpy(ada_base) for _ in range(blocks)]

    def act(rows, cols, r):
        return torch.from_numpy(S.activations(rows, cols, round(0.01 * cols), r).view(np.int16).copy()).view(
            torch.bfloat16).cuda()
    hid = S.STACK["hidden"]
    xq, xo, xu = (act(M, hid, rs[len(shapes) + 1 + i]) for i in range(3))
    xa = act(1, Ka, rs[len(shapes) + 4])
    ws = {k: torch.empty(max(layers[n][0].workspace_bytes(M) for n, kk, _ in shapes if kk == k),
                         dtype=torch.uint8, device="cuda") for k in {kk for _, kk, _ in shapes}}
    outs = {n: torch.empty((M, Nl), dtype=torch.bfloat16, device="cuda") for n, _, Nl in shapes}
    oa = torch.empty((1, Na), dtype=torch.bfloat16, device="cuda")
    k_of = {n: kk for n, kk, _ in shapes}
    g = [None]

    def svdq_pass():
        for b in range(blocks):
            layers["qkv"][b](xq, out=outs["qkv"], workspace=ws[k_of["qkv"]])
            layers["out"][b](xo, out=outs["out"], workspace=ws[k_of["out"]])
            layers["up"][b](xu, out=outs["up"], workspace=ws[k_of["up"]])
            g[0] = Fn.gelu(outs["up"])
            layers["down"][b](g[0], out=outs["down"], workspace=ws[k_of["down"]])

    def awq_pass():
        for b in range(blocks):
            ada[b](xa, out=oa)

    def full_pass():
        for b in range(blocks):
            ada[b](xa, out=oa)
            layers["qkv"][b](xq, out=outs["qkv"], workspace=ws[k_of["qkv"]])
            layers["out"][b](xo, out=outs["out"], workspace=ws[k_of["out"]])
            layers["up"][b](xu, out=outs["up"], workspace=ws[k_of["up"]])
            g[0] = Fn.gelu(outs["up"])
            layers["down"][b](g[0], out=outs["down"], workspace=ws[k_of["down"]])

    # the same blocks with the attention's per-head RMSNorm and RoPE on q and k:
    # as torch ops after the QKV linear, and with both fusions
    heads = hid // 128
    rq = rs[len(shapes) + 5]
    qn, kn = (torch.from_numpy(S.norm_weight(128, rq).view(np.int16).copy()).view(torch.bfloat16).cuda()
              for _ in range(2))
    cos, sin = (torch.from_numpy(t).cuda() for t in S.rope_tables(M, 128))
    ws_mlp = torch.empty(bq.mlp_workspace_bytes(M, layers["up"][0], layers["down"][0]), dtype=torch.uint8,
                         device="cuda")
    keep = [None]

    def unfused_pass():
        for b in range(blocks):
            ada[b](xa, out=oa)
            layers["qkv"][b](xq, out=outs["qkv"], workspace=ws[k_of["qkv"]])
            keep[0] = torch_norm_rope(outs["qkv"], heads, qn, kn, cos, sin)
            layers["out"][b](xo, out=outs["out"], workspace=ws[k_of["out"]])
            layers["up"][b](xu, out=outs["up"], workspace=ws[k_of["up"]])
            g[0] = Fn.gelu(outs["up"])
            layers["down"][b](g[0], out=outs["down"], workspace=ws[k_of["down"]])

    def fused_pass():
        for b in range(blocks):
            ada[b](xa, out=oa)
            bq.svdq_w4a4_qkv_rmsnorm_rope(xq, layers["qkv"][b], heads, qn, kn, cos, sin, out=outs["qkv"],
                                          workspace=ws[k_of["qkv"]])
            layers["out"][b](xo, out=outs["out"], workspace=ws[k_of["out"]])
            bq.svdq_w4a4_mlp_gelu(xu, layers["up"][b], layers["down"][b], out=outs["down"], workspace=ws_mlp)
    full_pass()
    unfused_pass()
    fused_pass()
    t_full = time_events(full_pass, passes, stream)
    t_svdq = time_events(svdq_pass, passes, stream)
    t_unf = time_events(unfused_pass, passes, stream)
    t_fus = time_events(fused_pass, passes, stream)
    t_awq = time_graph(awq_pass, passes, stream)
    if t_awq is None:
        t_awq = time_events(awq_pass, passes, stream)
    svdq_ops = blocks * sum(2.0 * M * Nl * Kl for _, Kl, Nl in shapes)
    awq_bytes = blocks * (Na * Ka // 2 + 2 * Na * (Ka // 64) * 2 + Ka * 2 + Na * 4)
    return {"blocks": blocks, "passes": passes, "pass_ms": round(t_full, 3),
            "svdq_and_gelu_pass_ms": round(t_svdq, 3), "awq_pass_ms": round(t_awq, 3),
            "svdq_TOPS_incl_gelu": round(svdq_ops / (t_svdq * 1e-3) / 1e12, 1),
            "awq_GBps": round(awq_bytes / (t_awq * 1e-3) / 1e9, 1),
            "with_norm_rope_pass_ms": round(t_unf, 3), "fused_pass_ms": round(t_fus, 3),
            "fused_speedup": round(t_unf / t_fus, 3),
            "svdq_ops_per_pass": svdq_ops, "awq_bytes_per_pass": awq_bytes}


def bench_mfma_peak(torch, stream, iters=20000):
    """Measured rate of v_mfma_f32_32x32x16_f16 (the product kernel's
    instruction): one 8-wave workgroup per CU, 8 independent accumulators per
    wave, once with each lane's operands fixed and once with operands that
    switch on every product (values like quantized data).  The chip's clock
    under sustained matrix load depends on how many operand bits switch, so
    the second figure is the ceiling that a product of real data meets.  The
    published dense peak (2.5 PFLOP/s) corresponds to 2.4 GHz; the clock
    implied by each measured rate is reported beside it."""
    import ctypes
    path = os.path.join(ROOT, "bit_quantized_linear_quantize_amd", "lib", "libsvdq_peak.so")
    if not os.path.exists(path):
        return None
    log("timing the matrix-instruction peak ...")
    lib = ctypes.CDLL(path)
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    flops = blocks * 8 * iters * 8 * 2.0 * 32 * 32 * 16
    out = {"instruction": "v_mfma_f32_32x32x16_f16", "published_dense_peak_TFLOPs": PEAK["f16"],
           "workgroups": blocks, "rounds_per_wave": iters}
    for key, name in (("fixed_operands", "svdq_peak_mfma_f16"), ("switching_operands", "svdq_peak_mfma_f16_switching")):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int

        def run():
            if fn(iters, blocks, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("peak probe launch failed")
        for _ in range(3):
            run()
        tflops = flops / (time_events(run, 5, stream) * 1e-3) / 1e12
        out[key] = {"measured_TFLOPs": round(tflops, 1), "implied_clock_GHz": round(2.4 * tflops / PEAK["f16"], 3)}
    # the other int4 datapath's inner loop: codes as fp8 / fp6 operands of the
    # 32x32x64 f8f6f4 instruction (one group per product) with the bf16 group
    # scales applied on the vector ALU
    fn = lib.svdq_peak_group_scaled
    fn.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    giters = iters // 4
    gflops = blocks * 8 * giters * 8 * 2.0 * 32 * 32 * 64
    for key, fmt in (("int4_as_fp8_group_scaled", 0), ("int4_as_fp6_group_scaled", 2)):
        def run():
            if fn(fmt, giters, blocks, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("group-scaled probe launch failed")
        for _ in range(3):
            run()
        out[key] = {"measured_TFLOPs": round(gflops / (time_events(run, 5, stream) * 1e-3) / 1e12, 1),
                    "instruction": "v_mfma_scale_f32_32x32x64_f8f6f4 + 2 VALU per output and group"}
    # the int4 product kernel's inner loop as built: per tile and group one
    # f8f6f4 product, one bf16 outer-product instruction for the scale
    # products and one FMA per output, on the kernel's 64 x 96 wave tile
    fn = lib.svdq_peak_outer_scaled
    fn.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    oiters = iters // 2
    oflops = blocks * 8 * oiters * 6 * 2.0 * 32 * 32 * 64
    for key, fmt in (("int4_as_fp8_outer_scaled", 0), ("int4_as_fp6_outer_scaled", 2)):
        def run():
            if fn(fmt, oiters, blocks, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("outer-scaled probe launch failed")
        for _ in range(3):
            run()
        out[key] = {"measured_TFLOPs": round(oflops / (time_events(run, 5, stream) * 1e-3) / 1e12, 1),
                    "instruction": "v_mfma_scale_f32_32x32x64_f8f6f4 + v_mfma_f32_32x32x8_bf16 (scale products) "
                                   "+ 1 FMA per output and group"}
    return out


def warm_clock(fn, seconds, torch):
    """Run fn back to back for at least `seconds` of wall time (the GPU clock
    ramps up under sustained load); returns the calls made."""
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(16):
            fn()
        n += 16
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_events(fn, steps, stream):
    """Per-call time of `steps` eager calls of fn, bracketed by events on
    `stream`.  One untimed call is queued before the start event, so the GPU
    is already busy while the host issues the first timed call."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    fn()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


def time_graph(calls, reps, stream, inner=1):
    """Per-call time of the launch sequence `calls` (library launches on the
    current stream only), captured `inner` times in a row into one HIP graph
    and replayed `reps` times, so that host launch cost stays out of the
    figure.  A graph launch itself costs the host tens of microseconds, so a
    sequence shorter than that needs `inner` > 1 to keep the GPU busy.
    Returns None if the capture fails (the caller then times eager calls)."""
    import torch
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(inner):
                calls()
        g.replay()
        torch.cuda.synchronize()
    except Exception as e:  # capture unavailable: eager launches
        log(f"graph capture failed ({e}); timing eager launches")
        return None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / (reps * inner)  # ms per captured sequence


ONLY_LEGS = {"quant_int4", "quant_nvfp4", "gemm_int4", "gemm_nvfp4", "awq_m1", "awq_m16", "mlp_fused", "qkv_fused",
             "copy"}


def run_only(leg, steps):
    """Launch a single kernel of the headline workload `steps` times (after one
    warm-up call), for per-kernel hardware-counter passes and kernel traces.  `mlp_fused` is the
    fused GELU MLP pair (nvfp4, M=4096, 3072 -> 12288 -> 3072, rank 32);
    `qkv_fused` the QKV projection 3072 -> 9216 with RMSNorm + RoPE (nvfp4).
    `copy` is a plain device-to-device copy of 256 MiB, the reference for
    scaling HBM byte counters."""
    import numpy as np
    import torch

    import synthetic as S
    import bit_quantized_linear_quantize_amd as bq

    bq.lib()
    torch.cuda.set_device(0)
    M, K, N, rank = 4096, 3072, 3072, 32
    if leg == "copy":
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        fn = lambda: b.copy_(a)
    elif leg.startswith("awq"):
        Ma = 1 if leg == "awq_m1" else 16
        ra = S.streams(7, 13)
        layers = [bq.AWQLinear.from_numpy(S.random_awq_layer(18432, 3072, ra[i])) for i in range(12)]
        xa = torch.from_numpy(S.activations(Ma, 3072, 0, ra[-1]).view(np.int16).copy()).view(torch.bfloat16).cuda()
        oa = torch.empty((Ma, 18432), dtype=torch.bfloat16, device="cuda")
        it = [0]

        def fn():
            layers[it[0] % 12](xa, out=oa)
            it[0] += 1
    elif leg == "mlp_fused":
        H = 12288
        r_up, r_dn = S.streams(11, 2)
        rx = S.streams(0, 2)[0]
        up = bq.SVDQLinear.from_numpy(S.random_svdq_layer(H, K, "nvfp4", rank, r_up))
        down = bq.SVDQLinear.from_numpy(S.random_svdq_layer(K, H, "nvfp4", rank, r_dn))
        x = torch.from_numpy(S.activations(M, K, round(0.01 * K), rx).view(np.int16).copy()).view(torch.bfloat16).cuda()
        ws = torch.empty(bq.mlp_workspace_bytes(M, up, down), dtype=torch.uint8, device="cuda")
        y = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        fn = lambda: bq.svdq_w4a4_mlp_gelu(x, up, down, out=y, workspace=ws)
    elif leg == "qkv_fused":
        heads, Nq = 24, 9216
        rl, rx, rn = S.streams(17, 3)
        layer = bq.SVDQLinear.from_numpy(S.random_svdq_layer(Nq, K, "nvfp4", rank, rl))
        x = torch.from_numpy(S.activations(M, K, round(0.01 * K), rx).view(np.int16).copy()).view(torch.bfloat16).cuda()
        qn, kn = (torch.from_numpy(S.norm_weight(128, rn).view(np.int16).copy()).view(torch.bfloat16).cuda()
                  for _ in range(2))
        cos, sin = (torch.from_numpy(t).cuda() for t in S.rope_tables(M, 128))
        ws = torch.empty(layer.workspace_bytes(M), dtype=torch.uint8, device="cuda")
        y = torch.empty((M, Nq), dtype=torch.bfloat16, device="cuda")
        fn = lambda: bq.svdq_w4a4_qkv_rmsnorm_rope(x, layer, heads, qn, kn, cos, sin, out=y, workspace=ws)
    else:
        # the headline legs' layer: the synthetic config-1 weight prepared on the GPU
        precision = "int4" if leg.endswith("int4") else "nvfp4"
        c1 = S.config1()
        x = torch.from_numpy(c1["x"].view(np.int16).copy()).view(torch.bfloat16).cuda()
        w1 = torch.from_numpy(c1["w"].astype(np.float32)).cuda()
        b1 = torch.from_numpy(c1["bias"].view(np.int16).copy()).view(torch.bfloat16).cuda()
        layer = bq.prepare_layer(w1, x, rank, precision, bias=b1)
        ws = torch.empty(layer.workspace_bytes(M), dtype=torch.uint8, device="cuda")
        bq.svdq_w4a4_quantize(x, layer, ws)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if leg.startswith("quant"):
            fn = lambda: bq.svdq_w4a4_quantize(x, layer, ws)
        else:
            fn = lambda: bq.svdq_w4a4_gemm(ws, M, layer, out=out)
    fn()
    torch.cuda.synchronize()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    log(f"ran {leg} x{steps}")


def layer_numpy(layer):
    """The oracle's dict form of a device SVDQLinear (bf16 as uint16 bits)."""
    import numpy as np
    import torch
    from oracle import formats as F

    def bits(t):
        return None if t is None else t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    p = layer.precision
    ws = bits(layer.wscales) if p == "int4" else layer.wscales.cpu().numpy()
    packed = layer.packed_w.cpu().numpy()
    return dict(precision=p, rank=layer.rank, packed_w=packed, w_codes=F.unpack_nibbles(packed), wscales=ws,
                wtscale=layer.wtscale, smooth=bits(layer.smooth),
                lora_down=bits(layer.lora_down) if layer.rank else np.zeros((0, layer.K), np.uint16),
                lora_up=bits(layer.lora_up) if layer.rank else np.zeros((layer.N, 0), np.uint16),
                bias=bits(layer.bias))


def cpu_baselines(S, np, x_bits, layers, budget):
    """The CPU oracle (numpy / OpenBLAS fp64) timed on bounded samples of
    configs 1-4: for each, calls repeat until about `budget` seconds (at least
    one), and the rate is scaled to the config's full workload."""
    from oracle import formats as F, layers as L
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count()

    def timed(fn, budget_s):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                return (time.perf_counter() - t0) / reps, reps
    M, K = x_bits.shape
    N = layers["int4"]["N"]
    out = {}
    for p in ("int4", "nvfp4"):
        dt, reps = timed(lambda: L.svdq_linear_ref(x_bits, layers[p]), budget)
        out[f"config_{1 if p == 'int4' else 2}_{p}"] = {
            "value": round(2.0 * M * N * K / dt / 1e12, 6), "unit": "TOPS", "seconds_per_call": round(dt, 3),
            "sample": f"the full workload ({M}x{K} activations, {N}x{K} {p} layer, rank 32), {reps} calls"}
    # config 3: AWQ adaLN linear 3072 -> 18432 at M = 1, 2, 16
    ra = S.streams(7, 2)
    awq = S.random_awq_layer(18432, 3072, ra[0])
    awq = dict(awq, q=F.unpack_nibbles(awq["packed_w"]), group_size=64)
    for Ma in (1, 2, 16):
        xa = S.activations(Ma, 3072, 0, ra[1])
        dt, reps = timed(lambda: L.awq_linear_ref(xa, awq), budget / 4)
        nbytes = 18432 * 3072 // 2 + 2 * 18432 * 48 * 2 + Ma * 3072 * 2 + Ma * 18432 * 2 + 18432 * 2
        out[f"config_3_awq_M{Ma}"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
                                      "seconds_per_call": round(dt, 4),
                                      "sample": f"the full layer 18432x3072 at M={Ma}, {reps} calls"}
    # config 4: one block's layers at full size, extrapolated to 24 blocks x 8 passes
    # (identical work per block and pass)
    rows = S.STACK["tokens"]
    rs = S.streams(13, len(S.STACK_LAYERS) + 1)
    blk, ops = 0.0, 0.0
    for i, (name, Kl, Nl) in enumerate(S.STACK_LAYERS):
        lay = S.random_svdq_layer(Nl, Kl, "nvfp4", 32, rs[i])
        lay = dict(lay, w_codes=F.unpack_nibbles(lay["packed_w"]))
        xl = S.activations(rows, Kl, round(0.01 * Kl), rs[-1])
        dt, _ = timed(lambda: L.svdq_linear_ref(xl, lay), 0.0)
        blk += dt
        ops += 2.0 * rows * Nl * Kl
    xa = S.activations(1, 3072, 0, ra[1])
    dt, _ = timed(lambda: L.awq_linear_ref(xa, awq), 0.0)
    blk += dt
    passes, blocks = S.STACK["passes"], S.STACK["blocks"]
    out["config_4_stack"] = {"value": round(ops / blk / 1e12, 6), "unit": "TOPS (svdq layers, block incl. adaLN)",
                             "extrapolated": True, "block_s": round(blk, 2), "pass_s": round(blk * blocks, 1),
                             "eight_passes_s": round(blk * blocks * passes, 1),
                             "sample": f"one block: its QKV, out, up and down linears (nvfp4, rank 32, {rows} "
                                       f"tokens) and its adaLN AWQ linear at M=1, one call each; the pass is "
                                       f"{blocks} such blocks and the config {passes} passes"}
    return out, threads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps after the wall-time warm-up")
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="wall time each timed leg runs untimed first, for the GPU clock to settle")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-budget", type=float, default=4.0, help="seconds of CPU oracle work per config sample")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the nvfp4, AWQ, MLP-pair and DiT-stack legs")
    ap.add_argument("--no-stack", action="store_true", help="skip the DiT-stack leg")
    ap.add_argument("--only", choices=sorted(ONLY_LEGS),
                    help="run one kernel --steps times and exit (for rocprofv3 counter passes)")
    args = ap.parse_args()
    if args.only:
        run_only(args.only, args.steps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU kernel path only: the library has no multi-GPU "
              "path (it would shard along tokens with replicated weights); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic as S
    import bit_quantized_linear_quantize_amd as bq

    bq.lib()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')}")

    M, K, N, rank = 4096, 3072, 3072, 32
    c1 = S.config1()
    x_bits = c1["x"]
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    w1 = torch.from_numpy(c1["w"].astype(np.float32)).cuda()
    b1 = torch.from_numpy(c1["bias"].view(np.int16).copy()).view(torch.bfloat16).cuda()
    ops = 2.0 * M * N * K
    log("preparing the config-1 layer on the GPU (int4 and nvfp4) ...")
    t0 = time.perf_counter()
    layers = {p: bq.prepare_layer(w1, x, rank, p, bias=b1) for p in ("int4", "nvfp4")}
    torch.cuda.synchronize()
    prep_s = (time.perf_counter() - t0) / 2

    def bench_svdq(precision, steps, warmup):
        layer = layers[precision]
        ws = torch.empty(layer.workspace_bytes(M), dtype=torch.uint8, device="cuda")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        G = bq.GROUP_SIZE[precision]
        step = lambda: layer(x, out=out, workspace=ws)
        k1 = lambda: bq.svdq_w4a4_quantize(x, layer, ws)
        k2 = lambda: bq.svdq_w4a4_gemm(ws, M, layer, out=out)
        # the two kernels alone, timed back to back through the C ABI with the
        # arguments marshalled once (the binding's per-call checks cost about
        # as much host time as kernel 1 takes on the GPU)
        L, P = bq.lib(), ctypes.c_void_p
        st = P(stream.cuda_stream)
        a1 = (P(x.data_ptr()), M, K, P(layer.smooth.data_ptr()), P(layer.lora_down.data_ptr()),
              bq.PRECISIONS[precision], G, rank, P(ws.data_ptr()), ws.numel(), st)
        a2 = (P(ws.data_ptr()), ws.numel(), M, K, N, P(layer.packed_w.data_ptr()), P(layer.wscales.data_ptr()),
              layer.wtscale, P(layer.lora_up.data_ptr()), P(layer.bias.data_ptr()), bq.PRECISIONS[precision], G,
              rank, P(out.data_ptr()), st)

        def raw1():
            if L.svdq_w4a4_quantize(*a1) != 0:
                raise RuntimeError("svdq_w4a4_quantize failed")

        def raw2():
            if L.svdq_w4a4_gemm(*a2) != 0:
                raise RuntimeError("svdq_w4a4_gemm failed")
        warm_clock(step, args.warm_seconds, torch)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        if torch.distributed.is_available() and torch.distributed.is_initialized():
            torch.distributed.barrier()
        ms = time_events(step, steps, stream)
        for _ in range(warmup):
            k1()
            k2()
        t1 = time_events(raw1, steps, stream)
        t2 = time_events(raw2, steps, stream)
        sb = 2 if precision == "int4" else 1
        # algorithmic bytes of kernel 1: read x, smooth, lora_down; write 4-bit codes
        # (counted at 4 bits although the workspace keeps int4 codes as fp8 bytes and
        # nvfp4 values as fp16), scales, lora_act
        k1_bytes = M * K * 2 + K * 2 + rank * K * 2 + M * K // 2 + M * (K // G) * sb + M * rank * 4
        return dict(ms=ms, k1_ms=t1, k2_ms=t2, k1_bytes=k1_bytes)

    log("timing svdq_w4a4 int4 ...")
    r4 = bench_svdq("int4", args.steps, args.warmup)
    value = ops / (r4["ms"] * 1e-3) / 1e12
    k2_tops = ops / (r4["k2_ms"] * 1e-3) / 1e12
    # the int4 product runs on fp8 matrix instructions (the codes are exact
    # E4M3 values, one group of 64 per instruction), with the bf16 group
    # scales applied per group, so its peak is the dense fp8 one
    roofline = {"kernel": "gemm_w4a4_lora_up<int4>", "bound": "mfma", "achieved": round(k2_tops, 2),
                "peak": PEAK["fp8"], "unit": "TFLOP/s", "frac": round(k2_tops / PEAK["fp8"], 4),
                "traffic": measured_traffic("gemm_w4a4_lora_up", "int4_4096x3072x3072_r32"),
                "avg_launch_us": round(r4["k2_ms"] * 1e3, 2),
                "instruction": "v_mfma_f32_32x32x64_f8f6f4 (int4 codes as fp8 E4M3) + v_mfma_f32_32x32x8_bf16 "
                               "(scale products s_x s_w) + 1 fp32 FMA per output and group",
                "frac_of_f16_peak": round(k2_tops / PEAK["f16"], 4)}

    extra = {"int4": {"step_us": round(r4["ms"] * 1e3, 2),
                      "quantize_act_lora_down_us": round(r4["k1_ms"] * 1e3, 2),
                      "quantize_act_lora_down_GBps": round(r4["k1_bytes"] / (r4["k1_ms"] * 1e-3) / 1e9, 1),
                      "gemm_w4a4_lora_up_us": round(r4["k2_ms"] * 1e3, 2),
                      "gemm_w4a4_lora_up_TOPS": round(k2_tops, 1)},
             "config1_layer_prepared_on_gpu_s": round(prep_s, 3)}

    if not args.no_extra:
        log("timing svdq_w4a4 nvfp4 ...")
        r8 = bench_svdq("nvfp4", args.steps, args.warmup)
        k2n = ops / (r8["k2_ms"] * 1e-3) / 1e12
        extra["nvfp4"] = {"value_TOPS": round(ops / (r8["ms"] * 1e-3) / 1e12, 1),
                          "step_us": round(r8["ms"] * 1e3, 2),
                          "quantize_act_lora_down_us": round(r8["k1_ms"] * 1e3, 2),
                          "quantize_act_lora_down_GBps": round(r8["k1_bytes"] / (r8["k1_ms"] * 1e-3) / 1e9, 1),
                          "gemm_w4a4_lora_up_us": round(r8["k2_ms"] * 1e3, 2),
                          "gemm_w4a4_lora_up_TOPS": round(k2n, 1),
                          "gemm_frac_of_f16_peak": round(k2n / PEAK["f16"], 4),
                          "instruction": "v_mfma_f32_32x32x16_f16 (exactly dequantized E2M1 x E4M3)"}
        # one GPU's share of the same layer when 8 GPUs split the tokens (M = 512):
        # 32 of the 256 x 192 tiles, so 1/8 of the CUs get work
        log("timing the M=512 token shard ...")
        xs = x[:512].contiguous()
        lay_s = layers["int4"]
        ws_s = torch.empty(lay_s.workspace_bytes(512), dtype=torch.uint8, device="cuda")
        out_s = torch.empty((512, N), dtype=torch.bfloat16, device="cuda")
        f_s = lambda: lay_s(xs, out=out_s, workspace=ws_s)
        warm_clock(f_s, args.warm_seconds / 4, torch)
        t_s = time_graph(f_s, 20, stream, inner=16)
        t_se = time_events(f_s, 200, stream)
        if t_s is None:
            t_s = t_se
        extra["int4_token_shard_M512"] = {"step_us": round(t_s * 1e3, 2),
                                          "eager_step_us": round(t_se * 1e3, 2),
                                          "TOPS": round(2.0 * 512 * N * K / (t_s * 1e-3) / 1e12, 1),
                                          "tiles": 2 * 16}
        log("timing awq_w4a16 ...")
        Na, Ka, copies = 18432, 3072, 12
        ra = S.streams(7, copies + 1)
        awq_layers = [bq.AWQLinear.from_numpy(S.random_awq_layer(Na, Ka, ra[i])) for i in range(copies)]
        awq = {}
        for Ma in (1, 2, 16):
            xa = torch.from_numpy(S.activations(Ma, Ka, 0, ra[-1]).view(np.int16).copy()).view(torch.bfloat16).cuda()
            oa = torch.empty((Ma, Na), dtype=torch.bfloat16, device="cuda")
            it = [0]

            def call():
                awq_layers[it[0] % copies](xa, out=oa)
                it[0] += 1
            warm_clock(call, args.warm_seconds / 4, torch)

            def seq():  # 4 rounds over the rotating copies
                for _ in range(4 * copies):
                    call()
            ms = time_graph(seq, max(2, args.steps // (4 * copies)) * 5, stream)
            if ms is not None:
                ms /= 4 * copies
            else:
                ms = time_events(call, max(args.steps, 10 * copies), stream)
            nbytes = Na * Ka // 2 + 2 * Na * (Ka // 64) * 2 + Ma * Ka * 2 + Ma * Na * 2 + Na * 2
            gbps = nbytes / (ms * 1e-3) / 1e9
            awq[f"M={Ma}"] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                              "frac_of_hbm": round(gbps / PEAK["hbm"], 4), "bytes": nbytes}
        extra["awq_w4a16_N18432_K3072"] = awq
        del awq_layers
        torch.cuda.empty_cache()

        peak = bench_mfma_peak(torch, stream)
        if peak:
            extra["mfma_peak"] = peak
            g8 = peak["int4_as_fp8_outer_scaled"]["measured_TFLOPs"]
            roofline["measured_inner_loop_peak"] = g8
            roofline["frac_of_measured_peak"] = round(k2_tops / g8, 4)
        extra["mlp_pair_nvfp4_3072_12288_3072"] = bench_mlp_pair(bq, S, torch, np, x, M, K, rank, stream)
        extra["qkv_rmsnorm_rope_nvfp4_3072_9216"] = bench_qkv(bq, S, torch, np, M, K, rank, stream)
        extra["weight_prep"] = bench_weight_prep(bq, S, torch, np, stream)
        torch.cuda.empty_cache()
        if not args.no_stack:
            extra["dit_stack_nvfp4"] = bench_stack(bq, S, torch, np, M, rank, stream)
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        lays = {p: layer_numpy(layers[p]) for p in ("int4", "nvfp4")}
        for p in lays:
            lays[p]["N"] = N
        per, threads = cpu_baselines(S, np, x_bits, lays, args.cpu_budget)
        head = per["config_1_int4"]
        cpu = {"value": head["value"], "unit": "TOPS", "cores": threads, "kind": "oracle",
               "seconds_per_call": head["seconds_per_call"],
               "sample": head["sample"] + ": activation quantizer + fp64 dequantized GEMM + low-rank + bias "
                                          "(numpy/OpenBLAS); other configs under per_config",
               "per_config": per}

    rec = {"metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r4["ms"], 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
           "data": "synthetic",
           "config": {"workload": "svdq_w4a4 int4 linear, M=4096 K=N=3072, rank 32, group 64 "
                                  "(DiT attention projection, 1% outlier channels; the synthetic config-1 "
                                  "weight prepared on the GPU)",
                      "M": M, "K": K, "N": N, "rank": rank, "group_size": 64, "precision": "int4",
                      "parallelism": "none (1 GPU)"},
           "warmup_wall_s_per_leg": args.warm_seconds,
           "roofline": roofline, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
