"""The boundary from C: include/mlp.h compiles as strict C99 (gcc -std=c99
-pedantic -Werror), a C program links against libmlp.so and its host-only
entry points answer without a GPU (tests/abi_c_check.c)."""
import os
import shutil
import subprocess

import pytest


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_is_c99_and_links(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not found")
    lib = os.path.join(ROOT, "mlp_gemm_softmax_amd", "libmlp.so")
    if not os.path.exists(lib):
        pytest.skip("libmlp.so not built (run __graft_entry__.build())")
    exe = str(tmp_path / "abi_c_check")
    libdir = os.path.dirname(lib)
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_c_check.c"), "-L", libdir, "-lmlp", "-Wl,-rpath," + libdir, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok: abi ")
