"""The C ABI's host code under the address and undefined-behaviour sanitizers: the host
tests (argument checks, status codes, descriptor layout, symbol table) run in a child
process against a build of the library whose host code is instrumented, with the sanitizer
runtime preloaded; any report aborts the child. CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "masked_scaled_dot_amd"))


def test_abi_host_tests_under_sanitizers():
    import build_host_sanitized as bhs
    rt = bhs.runtime()
    if rt is None:
        pytest.skip("no sanitizer runtime in this toolchain")
    lib = bhs.build()
    env = dict(os.environ, SA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import masked_scaled_dot_amd._lib as L, sys; "
            "assert L.LIB_PATH == sys.argv[1], L.LIB_PATH; print('loaded', L.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", code, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
