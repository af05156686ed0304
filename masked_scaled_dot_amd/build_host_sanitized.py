"""Build a copy of ``libsa.so`` whose host code (the C ABI layer, ``csrc/api.cpp``) carries
the address and undefined-behaviour sanitizers; the device code is the regular build's.

Usage: ``python masked_scaled_dot_amd/build_host_sanitized.py`` after ``build.py``. The
result is ``masked_scaled_dot_amd/_build/libsa_host_san.so``; load it in place of the
regular library with ``SA_LIBRARY=<path>``, preloading the sanitizer runtime
(``runtime()``) into a CPU-only process. Only host code is instrumented: the sanitizer
flags apply to the host compilation pass alone.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import build as _build  # noqa: E402  (the regular build: flags, sources, object folder)

LIB = os.path.join(_build.BUILD, "libsa_host_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def runtime() -> str | None:
    """Path of the sanitizer runtime to preload, or None if the toolchain has none."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build() -> str:
    objs = [os.path.join(_build.BUILD, s + ".o") for s in _build.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    api_obj = os.path.join(_build.BUILD, "api.cpp.san.o")
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [_build.HIPCC, *flags, *HOST_SAN, "-x", "hip", "-c", os.path.join(_build.CSRC, "api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for api.cpp:\n{r.stdout}\n{r.stderr}")
    cmd = [_build.HIPCC, "-shared", "-fPIC", f"--offload-arch={_build.ARCH}", *HOST_SAN, "-shared-libsan",
           api_obj, *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
