"""Host-sanitized build of the library, for CPU tests only.

The C ABI layer (kvarn_api.cpp: argument checks, plans, dispatch) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host
code only; the kernel translation units are the ordinary objects of
build.py.  The result, ``libkvarn_asan.so`` beside the package, is loaded
through KVARN_LIBRARY by a process that preloads the ASan runtime
(asan_runtime()); tests/test_abi_sanitized.py runs the ABI tests that way.
Never used on a GPU or by the product.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from kv_cache_quantization_seal_amd import build as B

ASAN_LIB = os.path.join(B.PKG, "libkvarn_asan.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang ASan runtime that the sanitized library links against."""
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("no clang ASan runtime under /opt/rocm/llvm")
    return libs[-1]


def build_sanitized(verbose: bool = False) -> str:
    B.build(changed_only=True)   # the kernel objects
    obj = os.path.join(B.BUILD, "asan_kvarn_api.o")
    cmd = [B.HIPCC, *B.FLAGS, "-O1", "-g", *HOST_SAN, "-c", os.path.join(B.CSRC, "kvarn_api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on kvarn_api.cpp (sanitized):\n" + r.stdout + r.stderr)
    objs = [obj] + [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "kvarn_api.cpp"]
    tmp = ASAN_LIB + ".tmp"
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN[:4], "-shared-libasan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed (sanitized):\n" + r.stdout + r.stderr)
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    build_sanitized(verbose=True)
    sys.exit(0)
