"""The host-only checks of the C ABI (tests/test_abi_cpu.py) run again against
a build of the ABI layer instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer: any invalid memory access or undefined behaviour
in validation, planning or table building aborts the run."""
import os
import shutil
import subprocess
import sys

import pytest

from orthogonalising_matrix_optimizer_amd import build_sanitized as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_checks_under_address_and_ub_sanitizers():
    lib = bs.build_sanitized()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=bs.env(), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
