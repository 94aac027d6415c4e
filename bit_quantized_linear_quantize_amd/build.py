"""Build the gfx950 HIP library (libsvdq_w4a4.so) in-tree with hipcc.

Every call recompiles.  Flags: gfx950 only; -ffp-contract=off so the
quantizer's fp32 products and quotients round exactly as written (FMAs are
explicit); packed-fp32 VALU instructions disabled.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libsvdq_w4a4.so")
# benchmark helper (measured matrix-instruction peak), not part of the layer's interface
PEAK_LIB = os.path.join(LIBDIR, "libsvdq_peak.so")
PEAK_SOURCES = ["mfma_peak.hip"]
BUILD = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.cpp", "quantize_act.hip", "gemm_w4a4.hip", "awq_gemv.hip", "weight_prep.hip", "prep_svd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose=False):
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(BUILD, exist_ok=True)
    # generated sources (the bf16 GELU table of the fused MLP epilogue)
    sys.path.insert(0, HERE)
    import gelu_bf16_gen
    gelu_bf16_gen.write(os.path.join(BUILD, "gelu_bf16_table.inc"))

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        # api.cpp is host code that also defines the static device scratch
        # of the allocation-free entry point, so it is compiled as HIP too
        lang = ["-x", "hip"] if src.endswith(".hip") or src == "api.cpp" else []
        _run([HIPCC] + FLAGS + ["-I", BUILD] + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PEAK_SOURCES))
    for lib, o in ((LIB, objs[:len(SOURCES)]), (PEAK_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + o)
        os.replace(tmp, lib)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
