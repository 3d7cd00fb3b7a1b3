"""Build libpisa.so for gfx950 with hipcc, in-tree (next to this file).

Usage: ``python -m sparse_attention_diffusion_pool_amd.build`` (or ``build()`` from Python).
Every source is compiled to an object under ``_build/`` in parallel, then linked.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpisa.so")
SOURCES = ["pisa_host.cpp", "stats.hip", "route.hip", "attend_bf16.hip", "attend_f32.hip", "probe.hip",
           "static_ws.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def _compile(src: str, obj: str, extra) -> str:
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(verbose: bool = False, jobs: int = 8, extra=()) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {}
        for s in SOURCES:
            obj = os.path.join(bdir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs[ex.submit(_compile, os.path.join(CSRC, s), obj, list(extra))] = s
        for f in cf.as_completed(futs):
            err = f.result()
            if verbose and err.strip():
                print(f"[{futs[f]}]\n{err}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


def build_host_sanitized() -> str:
    """A copy of libpisa whose host layer (pisa_host.cpp: plans, argument checks, dispatch) is
    built by g++ with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the kernels'
    objects from ``build()``. For CPU-side checks of the C ABI (the GPU code is not instrumented).
    Loading it needs the ASan runtime preloaded (``gcc -print-file-name=libasan.so``)."""
    bdir = os.path.join(PKG, "_build")
    sdir = os.path.join(bdir, "asan")
    os.makedirs(sdir, exist_ok=True)
    dev_objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in dev_objs):
        build()
    gxx = shutil.which("g++") or "g++"
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    host_obj = os.path.join(sdir, "pisa_host.o")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", *san, "-c", os.path.join(CSRC, "pisa_host.cpp"), "-o", host_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed:\n{' '.join(cmd)}\n{r.stderr}")
    out = os.path.join(sdir, "libpisa_asan.so")
    cmd = [gxx, "-shared", *san, "-o", out, host_obj, *dev_objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
