"""The public header is usable from plain C: a C11 program (tests/c/consumer.c) compiled by gcc
with warnings as errors, linked against libpisa.so, runs the host-only calls (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

from sparse_attention_diffusion_pool_amd import _lib as L

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_plain_c_consumer(tmp_path):
    assert os.path.exists(L.LIB_PATH), "libpisa.so is not built"
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(L.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic-errors",
           f"-I{os.path.join(ROOT, 'include')}", "-isystem", ROCM_INCLUDE,
           os.path.join(HERE, "c", "consumer.c"), "-o", str(exe),
           f"-L{libdir}", "-lpisa", f"-Wl,-rpath,{libdir}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "consumer ok" in run.stdout, run.stdout + run.stderr
