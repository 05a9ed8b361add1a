"""Build libdgq.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc.

    python -m quantized_paged_kv_dgq_amd.build      (or __graft_entry__.build())

Every source is compiled to an object in ``_build/`` (in parallel), then linked into
``quantized_paged_kv_dgq_amd/libdgq.so``.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdgq.so")
ARCH = os.environ.get("DGQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "decode.hip", "g64.hip", "compress.hip", "append.hip", "lifecycle.hip", "markers.hip", "pool.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Werror", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# HIP device code: gfx950 only; packed FP32 instructions are kept out of generated code.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [_hipcc(), *HIP_FLAGS, *COMMON, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = ["g++", *COMMON, f"-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
