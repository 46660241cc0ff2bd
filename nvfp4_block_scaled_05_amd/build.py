"""Build ``libnvfp4.so`` (gfx950 only) in-tree with hipcc.

Flags that matter for the numerics:
  -ffp-contract=off   no fused multiply-add anywhere: every step of the scale
                      chain is one correctly rounded FP32 operation;
  (default)           correctly rounded FP32 division, IEEE denormals;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed FP32 instructions are generated.

For the matrix-core RHT transform, -mllvm -amdgpu-mfma-vgpr-form keeps MFMA
results in ordinary VGPRs (otherwise they land in accumulation registers
and every value costs a copy before the vector ALU can use it).
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnvfp4.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "amax.hip", "cast.hip", "rowscaled.hip", "dequant.hip", "swizzle.hip", "hooks.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC, "-Wall",
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(force: bool = True) -> str:
    """Compile every source and link the shared library; returns its path."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
        newest = max(newest, os.path.getmtime(os.path.join(INCLUDE, "nvfp4.h")))
        if os.path.getmtime(LIB) >= newest:
            return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
