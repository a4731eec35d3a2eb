"""Build libringattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m long_context_blockwise_amd.build      # or build() from Python

Every source is compiled on each call (the build is the "does it compile"
check); objects go to ``_build/`` next to this file and the library to
``libringattn.so`` in the package directory.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libringattn.so")
ARCH = os.environ.get("RING_ATTN_ARCH", "gfx950")

SOURCES = ["attn_fwd_bf16.hip", "attn_fwd_f32.hip", "attn_bwd_bf16.hip", "merge.hip", "stage_check.hip",
           "ring_attn.cpp"]

# Packed-fp32 VALU forms are disabled in all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          f"-I{INCLUDE}"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; that warning is expected
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
