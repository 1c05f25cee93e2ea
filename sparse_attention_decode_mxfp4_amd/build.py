"""Builds libmxsparse.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_attention_decode_mxfp4_amd.build

Every HIP source is compiled with hipcc for gfx950 only. Packed fp32 VALU
instructions are disabled (-packed-fp32-ops) and fp32 division and square
root are correctly rounded (the FP8 row store divides by its per-token scale).
The target feature reaches the host pass too, which warns that it does not
know it and ignores it: clang's -Xarch_device passes no option that takes an
argument, so -Xclang -target-feature cannot be limited to the device pass.
MFMA results go to VGPRs (-amdgpu-mfma-vgpr-form): the kernels read every
accumulator with VALU code, which AGPR results would first have to copy out.
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
LIB = os.path.join(PKG, "libmxsparse.so")
SOURCES = ["api.cpp", "store.hip", "score.hip", "topk.hip", "attn.hip", "merge.hip", "read.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
