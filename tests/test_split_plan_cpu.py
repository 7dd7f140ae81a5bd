"""The Hessian's token-split placement, replayed on the CPU.

`split_plan.hpp` (the same header the SYRK kernel and its reduction include)
is compiled with the host compiler into `split_plan_check`, which checks for
each shape that every (tile, split) is computed exactly once, with the split
count and length the reduction assumes, covering all tokens.  The mixed plan
only changes where the sum over tokens is cut ("GPTQ: Mathematical
Foundations ...", Second-Order Taylor Expansion and the Hessian: H is a sum
over tokens), so this host check plus the GPU Hessian parity tests cover it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "split_plan_check.cpp")
INC = os.path.join(ROOT, "post_weight_quantization_16_amd", "csrc")

CASES = [(4096, 131072, 7), (8192, 262144, 7), (8192, 131072, 3), (4096, 16384, 7),
         (2048, 65536, 7), (3072, 40000, 5), (16384, 131072, 2), (12288, 131072, 4),
         (4096, 131072, 2), (1024, 8192, 4), (8192, 262144, 5), (4096, 65536, 6)]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "split_plan_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-I", INC, SRC, "-o", exe], check=True)
    return exe


def test_every_tile_split_runs_once(checker):
    args = [str(v) for case in CASES for v in case]
    out = subprocess.run([checker, *args], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert out.stdout.count("mixed plan ok") >= 3   # the plan is exercised, not only the fallback
