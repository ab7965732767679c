"""Build libtq.so (the C-ABI library) in-tree with hipcc for gfx950.

Sources are compiled in parallel to objects under _build/ and linked into
kv_cache_vector_randomized_amd/libtq.so; the plain streaming kernels of the
benchmark's memory ceilings go to libtqstream.so.  Every call rebuilds.
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
OUT = os.path.join(PKG, "libtq.so")
STREAM_OUT = os.path.join(PKG, "libtqstream.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["tq_host.cpp", "tq_append.hip", "tq_decode.hip", "tq_dequant.hip", "tq_transfer.hip", "tq_polar.hip",
           "tq_generic.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found")
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, OUT)
    # the plain streaming kernels bench.py measures the memory ceilings with (not part of tq.h)
    tmp = STREAM_OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "stream_probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for stream_probe.hip:\n{r.stderr[-4000:]}")
    os.replace(tmp, STREAM_OUT)
    if verbose:
        print(f"built {OUT} and {STREAM_OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
