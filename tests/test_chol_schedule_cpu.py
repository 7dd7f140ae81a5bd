"""Host-side schedule of the Cholesky trailing updates (chol_sched.hpp).

The C++ checker (chol_sched_check.cpp) replays the schedule at 64x64-block
granularity: every block below the diagonal must receive every earlier
panel's rank-64 update exactly once, before the launch that factors its
panel; what one launch's workgroups write must be disjoint; every update
may read only finished panels.  Sizes cover the empty cases (one and two
super-panels), ragged edges and the benchmark layer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_16_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "chol_sched_check.cpp")

SIZES = [1, 63, 64, 65, 100, 128, 192, 255, 256, 257, 320, 384, 500, 640, 1000, 1024,
         1536, 2047, 2048, 3000, 4033, 4096, 5120]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("sched") / "chol_sched_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe], check=True)
    return exe


def test_schedule_covers_every_update_once(checker):
    out = subprocess.run([checker] + [str(d) for d in SIZES], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = out.stdout.strip().splitlines()
    assert len(lines) == len(SIZES) and all(l.startswith("ok ") for l in lines)


def test_schedule_spreads_the_far_work(checker):
    # 4096: 32 row tiles of 128; tile (r, t) takes the t−1 super-panels left of
    # its column tile (4960 rank-128 updates), mostly in pairs (a pair costs
    # 1.5 singles); no launch may cost more than 1.5x the average over the 59
    # launches that can hold far work plus the one task that crosses the
    # target, and the pairing halves the task count
    out = subprocess.run([checker, "4096"], capture_output=True, text=True, check=True).stdout
    fields = dict(f.split("=") for f in out.split()[1:])
    assert int(fields["far_updates"]) == 4960
    assert int(fields["far_tasks"]) <= 2600
    cost, peak = int(fields["cost"]), int(fields["peak_cost"])
    assert peak <= -(-3 * cost // (2 * 59)) + 3
