"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
on the CPU: tests/host_abi/ builds the sources with the sanitizers on their
host code, links them with a host stand-in of the HIP runtime and a check
program that drives every entry point (argument checks, workspace and scratch
carving, paged-table checks, launch planning over seeded random shapes up to
the largest batch, allocation failures inside create), and runs it. Any
sanitizer report aborts the program; any failed check makes it exit 1."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "host_abi"))

pytestmark = pytest.mark.timeout(600)


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")), reason="needs hipcc")
def test_host_code_is_clean_under_asan_and_ubsan():
    from build_check import build_check
    exe = build_check()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe, "160"], capture_output=True, text=True, env=env, timeout=500)
    report = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, report
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " 0 failures" in r.stdout, report
    print(r.stdout.strip())
