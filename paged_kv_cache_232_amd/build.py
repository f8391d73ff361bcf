"""Build the HIP library libpkv.so for gfx950 in-tree with hipcc.

Usage: python -m paged_kv_cache_232_amd.build   (or call build()).
Every call recompiles every source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["api.cpp", "noalloc.cpp", "cache.hip", "decode.hip", "prefill.hip", "blocks.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code (hipcc -O3 would otherwise form them
# from plain float code). MFMA results are kept in VGPR form: with the accumulator-register form
# the allocator copied the whole output accumulator between AGPRs and VGPRs on every loop
# iteration of the head_dim-256 kernels.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
            cmd = [hipcc, *HIP_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libpkv.so")
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        shutil.move(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
