"""The statistics passes' split of the (head, block) pairs into workgroup ranges, and the partial
slots the finalize kernel sums per head, checked exhaustively on small shapes and on the
benchmark layers' shapes (tests/c/stat_ranges.cpp, built with g++ against the kernels' internal
header; host code only)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "sparse_attention_diffusion_pool_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_stat_ranges(tmp_path):
    exe = tmp_path / "stat_ranges"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}",
           "-isystem", "/opt/rocm/include", os.path.join(HERE, "c", "stat_ranges.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and "ranges ok" in run.stdout, run.stdout + run.stderr
