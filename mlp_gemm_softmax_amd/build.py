"""Build ``libmlp.so`` (the C-ABI library) from ``csrc/`` with hipcc for gfx950.

Run ``python -m mlp_gemm_softmax_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``mlp_gemm_softmax_amd/_build/``; the library is written next to
this file so that it travels with the source tree.

``build_host_sanitized()`` (``python -m mlp_gemm_softmax_amd.build --host-sanitizers``)
builds ``libmlp_hostsan.so``: the same sources with the host code under
AddressSanitizer and UndefinedBehaviorSanitizer (``-Xarch_host`` only: the GPU
code is built as usual).  It is for host-side checks without a GPU -- argument
preflight and the checkpoint parser, which reads caller-supplied bytes -- and
needs the sanitizer runtime preloaded (``sanitizer_runtime()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmlp.so")
BUILD_DIR = os.path.join(HERE, "_build")
OUT_SAN = os.path.join(HERE, "libmlp_hostsan.so")
BUILD_DIR_SAN = os.path.join(HERE, "_build_hostsan")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # Packed fp32 VALU forms stay off: only plain v_fma/v_add forms are emitted.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmlp.so)")


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _build(out: str, build_dir: str, extra=(), verbose: bool = True, jobs: int | None = None) -> str:
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(len(sources), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), sources))
    tmp = out + ".tmp"
    libsan = ["-shared-libsan"] if extra else []   # the sanitizer runtime as a shared library
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *libsan, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(sources)} sources")
    return out


def build(verbose: bool = True, jobs: int | None = None) -> str:
    """Compile every source in csrc/ and link libmlp.so; returns its path."""
    return _build(OUT, BUILD_DIR, (), verbose, jobs)


def build_host_sanitized(verbose: bool = True, jobs: int | None = None) -> str:
    """libmlp_hostsan.so: host code under ASan + UBSan; returns its path."""
    return _build(OUT_SAN, BUILD_DIR_SAN, SAN_FLAGS, verbose, jobs)


C_CLIENT_SRC = os.path.join(ROOT, "tests", "abi_c_step.c")
C_CLIENT = os.path.join(HERE, "c_client_step")


def build_c_client(verbose: bool = True) -> str | None:
    """Compile the C test client of the ABI (``tests/abi_c_step.c``: a training
    step driven from C with hipMalloc'd memory) next to libmlp.so, which it
    links through an ``$ORIGIN`` rpath; returns its path, or None without gcc."""
    cc = shutil.which("gcc")
    if cc is None:
        if verbose:
            print("gcc not found: C test client not built")
        return None
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(rocm, "include"), f"-I{os.path.join(ROOT, 'include')}", C_CLIENT_SRC,
           f"-L{HERE}", "-lmlp", f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", C_CLIENT]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {C_CLIENT}")
    return C_CLIENT


def sanitizer_runtime() -> str | None:
    """Path of the AddressSanitizer runtime of ROCm's clang (to preload into
    a process that loads libmlp_hostsan.so), or None."""
    pats = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return sorted(pats)[-1] if pats else None


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv[1:]:
        build_host_sanitized()
    else:
        build()
        build_c_client()
    sys.exit(0)
