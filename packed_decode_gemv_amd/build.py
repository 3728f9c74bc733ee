"""Builds libvbq.so (HIP, gfx950) in-tree with hipcc.

Usage: python packed_decode_gemv_amd/build.py   (or call build()). It imports
only the standard library, so it runs before the library exists; importing
the package instead would load the library first.
Every source is compiled each time build() runs; objects go to _build/.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libvbq.so")
OBJ_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
    # packed-fp32 VALU ops are kept off (hipcc's host pass warns that it does
    # not know the feature; that is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]
# Sources whose arithmetic decides integers are built without FMA contraction.
EXACT = {"pack.hip", "verify.hip"}
SOURCES = ["api.cpp", "pack.hip", "gemv.hip", "verify.hip", "gemm.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src + ".o")
    flags = list(COMMON)
    flags.append("-ffp-contract=off" if src in EXACT else "-ffp-contract=fast")
    if src.endswith(".cpp"):
        flags = ["-x", "hip"] + flags
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
