"""The host code of libkvc under AddressSanitizer: the library is rebuilt with
the host side instrumented (device code untouched) and the host-only tests --
argument checks of every entry point, workspace sizing, the host control
routines -- run against it in a child process with the sanitizer runtime
preloaded. Any invalid host access aborts that process and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_code_under_address_sanitizer():
    from budgeted_retention_amd import build
    lib = build.build(asan=True)
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), KVC_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_abi_host.py", "tests/test_host_control.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "passed" in res.stdout and "AddressSanitizer" not in res.stderr
