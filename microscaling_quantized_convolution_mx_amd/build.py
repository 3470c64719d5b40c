"""Build step of the HIP library: compiles csrc/ for gfx950 into libmxconv.so.

Each translation unit is compiled in its own hipcc process (in parallel) and
linked into one shared object next to this file.  Flags:
  -ffp-contract=off        every fp32 step of the quantizer is one IEEE op
  -packed-fp32-ops off     no packed fp32 instructions are generated
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxconv.so")
ARCH = os.environ.get("MXCONV_ARCH", "gfx950")

SOURCES = ["capi.cpp", "quantize.hip", "quantize_mx.hip", "conv.hip", "conv_staged.hip", "conv8.hip", "conv_mixed.hip", "conv_mx.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if warn:
            sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every HIP translation unit and link libmxconv.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
