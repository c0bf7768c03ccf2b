"""CPU test of the 4-head group tiles (tril_solve_amd/csrc/tril_group.h).

tests/group_layout_check.cpp runs the header's own arithmetic on the host for
every plan the solver kernels use (fused, split diagonal, split merge) and
every input element type: where each lane of each direct-to-LDS load puts
which bytes of A (no overlaps, every held byte loaded once, nothing past the
tile), that every byte the solve reads through the address function is the
element it stands for, and that the 16 lanes of each read group fall on
different LDS banks. Planting a mistake in the header (the head rotation on
either side, or the slot padding) makes it fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def test_group_layout(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "group_layout_check")
    cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-std=c++20", "-O1",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "tril_solve_amd", "csrc"),
           os.path.join(ROOT, "tests", "group_layout_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    lines = run.stdout.strip().splitlines()
    assert lines[-1] == "ok"
    assert len(lines) == 8  # seven plans and "ok"
