"""The C-ABI host paths under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the host
layer is rebuilt by g++ with both sanitizers (``build.build_host_sanitized``), and the host API
tests (tests/test_api_host.py) run against that library in a fresh interpreter with the ASan
runtime preloaded. Any memory error or undefined behaviour in plan handling, argument checks or
status reporting aborts the run."""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

DRIVER = """
import sys
from sparse_attention_diffusion_pool_amd import _lib
_lib.load(sys.argv[1])
import pytest
sys.exit(pytest.main([sys.argv[2], "-q", "-p", "no:cacheprovider", "-m", "not gpu"]))
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_host_api_under_asan_and_ubsan():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-path check: runs where no GPU is visible")
    from sparse_attention_diffusion_pool_amd import build as b
    lib = b.build_host_sanitized()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), asan
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", DRIVER, lib, os.path.join(HERE, "test_api_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
