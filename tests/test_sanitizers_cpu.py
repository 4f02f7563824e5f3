"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the CPU tests of the ABI (argument preflight, the checkpoint parser fed
well-formed, damaged and random bytes) run against libmlp_hostsan.so in a
child process with the sanitizer runtime preloaded; any invalid access or
undefined behaviour ends that process with an error report."""
import os
import subprocess
import sys

import pytest

from mlp_gemm_softmax_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_code_is_clean_under_asan_and_ubsan():
    rt = build.sanitizer_runtime()
    if not os.path.exists(build.OUT_SAN) or rt is None:
        pytest.skip("libmlp_hostsan.so not built (python -m mlp_gemm_softmax_amd.build --host-sanitizers)")
    # the library is instrumented (ASan reports come from its own code)
    syms = subprocess.run(["nm", "-D", build.OUT_SAN], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_abi.py")], env=env,
                         capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
