"""Host-sanitised build of the C ABI (AddressSanitizer + UndefinedBehaviorSanitizer).

The ABI layer (validation, planning, descriptor tables, launch sequencing) is
plain host C++: it is compiled here with g++ and the sanitizers, and linked
with the device objects of the normal build (built first if missing) into
_build/sanitized/libmuon_mi355x_sanitized.so.  The kernels themselves are not
instrumented.  Load it by setting MUON_LIB_PATH to that file, with the
sanitizer runtime preloaded (see `env()`).

Usage: python -m orthogonalising_matrix_optimizer_amd.build_sanitized
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as _build

OUT_DIR = os.path.join(_build.BUILD, "sanitized")
LIB = os.path.join(OUT_DIR, "libmuon_mi355x_sanitized.so")
HOST_SOURCES = ["muon_api.cpp"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stderr)


def runtime() -> str:
    """Path of the AddressSanitizer runtime to preload."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def env() -> dict:
    """Environment for a process that loads the sanitised library."""
    e = dict(os.environ)
    pre = runtime()
    e["LD_PRELOAD"] = pre + (" " + e["LD_PRELOAD"] if e.get("LD_PRELOAD") else "")
    e["MUON_LIB_PATH"] = LIB
    # the interpreter's own allocations are not ours to report
    e["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    e["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return e


def build_sanitized() -> str:
    dev_objs = [os.path.join(_build.BUILD, os.path.splitext(s)[0] + ".o")
                for s in _build.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in dev_objs):
        _build.build()
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(ROCM, "include"), "-I", os.path.join(_build.ROOT, "include"),
              *SANITIZE, "-c", os.path.join(_build.CSRC, src), "-o", obj])
        objs.append(obj)
    _run(["g++", "-shared", *SANITIZE, "-o", LIB, *objs, *dev_objs,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
    sys.exit(0)
