"""Build libgptq_mi355x.so in-tree with hipcc for gfx950.

    python -m post_weight_quantization_16_amd.build

Sources are compiled in parallel into ``_build/`` next to this file and
linked into ``libgptq_mi355x.so`` beside it.  Every call rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgptq_mi355x.so")
ARCH = "gfx950"

# (source, object, extra flags); the sweep is built once per group-size variant
SOURCES = [
    ("api.hip", "api.o", []),
    ("gemm.hip", "gemm.o", []),
    ("hessian.hip", "hessian.o", []),
    ("prepare.hip", "prepare.o", []),
    ("quantize.hip", "quantize.o", []),
    ("export.hip", "export.o", []),
    ("obq.hip", "obq.o", []),
    ("timing.hip", "timing.o", []),
    ("w4a16.hip", "w4a16.o", []),
] + [("sweep.hip", f"sweep_g{g}.o", [f"-DGQ_SWEEP_G={g}"]) for g in (0, 32, 64, 128)]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"),
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the sweep fully unrolls its 128-column loop so the block stays in VGPRs
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-Wno-pass-failed",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, o) for _, o, _ in SOURCES]
    jobs = [[hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", os.path.join(BUILD, o)]
            for src, o, extra in SOURCES]
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 4, 16)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
