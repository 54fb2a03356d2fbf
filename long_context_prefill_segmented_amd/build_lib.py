"""Builds libdhsa.so in-tree with hipcc for gfx950 (no CUDA, no other target).

    python -m long_context_prefill_segmented_amd.build_lib
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdhsa.so")

SOURCES = ["dhsa_api.hip", "pool.hip", "scores.hip", "topk.hip", "attn.hip", "nms.hip", "layer.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source and link libdhsa.so; returns the library path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="dhsa_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libdhsa.so")
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
