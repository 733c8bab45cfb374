"""The C ABI under host sanitizers (CPU only): kla_api.hip's host code
(argument validation, workspace layouts, launch set-up) is built with
AddressSanitizer and UBSan for the host side, every kernel object unchanged,
and tests/test_abi.py runs against that library in a fresh process with the
ASan runtime preloaded.  Any sanitizer report fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_abi_under_host_sanitizers():
    sys.path.insert(0, os.path.join(ROOT, "bius_scan_sequence_amd"))
    try:
        import build as B
    finally:
        sys.path.pop(0)
    lib = B.build_host_sanitized()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in out and "__ubsan_" in out, "library not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.asan_runtime(), BIUS_KLA_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, log
    assert " passed" in r.stdout, log
