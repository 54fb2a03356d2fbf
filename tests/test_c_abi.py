"""The C ABI from a plain C program: tests/c/abi_check.c is compiled with gcc
against include/dhsa.h and linked to libdhsa.so; it runs only host-side calls
(size queries and argument checks), so it needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "long_context_prefill_segmented_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.skipif(not os.path.exists(os.path.join(LIBDIR, "libdhsa.so")),
                    reason="libdhsa.so not built")
def test_plain_c_client(tmp_path):
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", LIBDIR, "-ldhsa",
           f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    # the library's HIP runtime is resolved by the loader; no device is opened
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert res.returncode == 0, res.stderr
    assert "c abi ok" in res.stdout
