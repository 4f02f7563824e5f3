"""Runs tests/test_abi_cpu.py against libmlp_hostsan.so (the library with its
host code under AddressSanitizer and UBSan).  Started as a child process by
tests/test_sanitizers_cpu.py with the sanitizer runtime preloaded; not a test
module itself."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mlp_gemm_softmax_amd import binding, build  # noqa: E402

binding._LIB = binding.load_library(build.OUT_SAN)

import pytest  # noqa: E402

sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_cpu.py")]))
