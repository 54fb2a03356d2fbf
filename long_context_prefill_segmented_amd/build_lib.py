"""Builds libdhsa.so in-tree for gfx950 (no CUDA, no other target).

    python -m long_context_prefill_segmented_amd.build_lib

Each source compiles in two passes, as hipcc's own single pass does
internally: the device pass (gfx950 code object, bundled as a fat binary)
and the host pass, which embeds that fat binary.  Splitting them lets the
device-only flags (the packed-fp32 VALU forms switched off) reach the device
compiler alone, so the host compiler never sees an unknown target feature.
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

# bench.py's streaming-read reference (a measuring aid, not part of libdhsa)
BENCH_CSRC = os.path.join(PKG, "csrc_bench")
BENCH_LIB = os.path.join(PKG, "libdhsa_bench.so")
BENCH_SOURCES = ["hbm_read.hip"]

COMMON_FLAGS = [
    "-x", "hip",
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall", "-Wno-unused-function",
]
# device pass only: packed fp32 VALU forms are kept out of the device code
DEVICE_FLAGS = ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["--cuda-host-only"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def clang() -> str:
    """The HIP compiler driver hipcc itself runs (clang++ -x hip)."""
    for cand in (os.environ.get("HIP_CLANG"), "/opt/rocm/lib/llvm/bin/clang++"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("/opt/rocm/lib/llvm/bin/clang++ not found")


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{res.stdout}\n{res.stderr}")
    return res


def _build_lib(srcdir, sources, lib, verbose):
    cc, hc = clang(), hipcc()
    inc = ["-I", INCLUDE, "-I", srcdir]
    with tempfile.TemporaryDirectory(prefix="dhsa_build_") as tmp:
        objs = []
        for src in sources:
            path = os.path.join(srcdir, src)
            fatbin = os.path.join(tmp, src.replace(".hip", ".fatbin"))
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            _run([cc, *COMMON_FLAGS, *DEVICE_FLAGS, *inc, "-c", path, "-o", fatbin],
                 f"device pass of {src}", verbose)
            _run([cc, *COMMON_FLAGS, *HOST_FLAGS, *inc, "-Xclang", "-fcuda-include-gpubinary",
                  "-Xclang", fatbin, "-c", path, "-o", obj], f"host pass of {src}", verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, os.path.basename(lib))
        _run([hc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib], "link",
             verbose)
        os.replace(tmp_lib, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every source and link libdhsa.so (and bench.py's reference
    library libdhsa_bench.so); returns the path of libdhsa.so."""
    _build_lib(BENCH_CSRC, BENCH_SOURCES, BENCH_LIB, verbose)
    return _build_lib(CSRC, SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
