"""Build libq2kdecode.so in-tree with hipcc for gfx950.

Every HIP source is compiled to an object (in parallel) under ``_build/``
and linked into ``q2_quantized_decode_amd/libq2kdecode.so``. Flags: -O3, no
fast-math (the q8_1 quantiser relies on correctly rounded f32 division), and
packed FP32 instructions disabled for device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq2kdecode.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "mmvq.hip", "mmvq_mfma.hip", "mmq.hip", "gemv_bf16.hip", "q8_1.hip", "engram.hip"]

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Kernel-argument preloading: the leading scalar arguments of every kernel
# (up to 16 SGPRs) are loaded into SGPRs at wave launch instead of by the
# wave's first scalar loads. The code object keeps a fallback entry that
# loads them, used where the firmware does not preload.
DEVICE_FLAGS += ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
SOURCE_FLAGS: dict = {}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
