"""Build libkvarn.so (HIP, gfx950) in-tree with hipcc.

Each source compiles to an object in ``_build/`` (in parallel), then one link
step produces ``kv_cache_quantization_seal_amd/libkvarn.so``.  The read probe
(a measurement aid with no KVarN computation) links into its own
``libkvarn_probe.so``.  Packed fp32 instructions are disabled for every HIP
translation unit.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvarn.so")
PROBE_LIB = os.path.join(PKG, "libkvarn_probe.so")
TRACE_LIB = os.path.join(PKG, "libkvarn_trace.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["kvarn_api.cpp", "seal.hip", "decode.hip", "cache.hip", "prefill_attn.hip",
           "decode_k2.hip", "decode_k3.hip", "decode_k4.hip", "decode_k5.hip", "decode_k6.hip", "decode_k8.hip"]
PROBE_SOURCES = ["read_probe.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]
# Decode inputs are finite by contract: with NaNs not honoured and the IEEE
# mode bit off, float max/min need no quieting of their operands.
EXTRA = {s: ["-fno-honor-nans", "-mno-amdgpu-ieee"] for s in SOURCES if s.startswith("decode")}


def _compile(src: str, trace: bool = False) -> str:
    obj = os.path.join(BUILD, ("trace_" if trace else "") + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *(["-DKVARN_WAVE_TRACE"] if trace else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def _stale(src: str) -> bool:
    """True if src's object is missing or older than src or any header."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".hpp")]
    deps.append(os.path.join(ROOT, "include", "kvarn.h"))
    return max(os.path.getmtime(p) for p in deps) > os.path.getmtime(obj)


def build(verbose: bool = False, changed_only: bool = False) -> str:
    """Compile every source (or, with changed_only, those whose object is
    older than the source or a header) and link both libraries."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    todo = [s for s in srcs if _stale(s)] if changed_only else srcs
    objs = {s: os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs}
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(len(todo), os.cpu_count() or 1))) as ex:
        list(ex.map(_compile, todo))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


def build_trace(verbose: bool = False) -> str:
    """The trace build: the same sources with per-wave phase timestamps
    compiled in (KVARN_WAVE_TRACE), linked as libkvarn_trace.so.  A
    diagnostic library, never loaded unless asked for (KVARN_LIBRARY)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, trace=True), SOURCES))
    _link(objs, TRACE_LIB)
    if verbose:
        print(f"built {TRACE_LIB}")
    return TRACE_LIB


if __name__ == "__main__":
    if "--trace" in sys.argv:
        build_trace(verbose=True)
    else:
        build(verbose=True, changed_only="--changed" in sys.argv)
