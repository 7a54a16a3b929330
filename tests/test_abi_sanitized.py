"""The ABI tests (tests/test_abi.py: exports, argument validation before any
launch, sizes and plans; no GPU needed) against a build of the library whose
host code runs under AddressSanitizer and UndefinedBehaviorSanitizer, in a
child process that preloads the ASan runtime.  Any sanitizer report fails
the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers():
    from kv_cache_quantization_seal_amd import build_sanitize as S
    try:
        lib = S.build_sanitized()
        rt = S.asan_runtime()
    except (RuntimeError, OSError) as e:   # no hipcc or ASan runtime in this environment
        pytest.skip(f"sanitized build unavailable: {e}")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, KVARN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
