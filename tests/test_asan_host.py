"""The host side of the C ABI (descriptor, size, segment-table and overlap
checks, workspace queries, the Python binding's buffer checks) run against a
build whose host code is under AddressSanitizer. The three ABI test files run
in a child process with the sanitizer runtime preloaded; any heap or stack
error the checks make aborts that process. No kernel is launched."""
import os
import subprocess
import sys

import pytest

from linear_recurrent_lm_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suites_under_address_sanitizer():
    try:
        runtime = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_asan()
    env = dict(os.environ, LD_PRELOAD=runtime, WKV7_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    files = ["tests/test_abi.py", "tests/test_vce_abi.py", "tests/test_binding_validation.py"]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", *files], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr, tail
    assert " passed" in res.stdout, tail
