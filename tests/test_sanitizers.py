"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with host code instrumented (device code as in the normal build),
then runs the ABI and schedule suites against it in a child process with the ASan
runtime preloaded: every argument check, size computation, error path, workspace
formula and schedule query of the C-ABI runs instrumented, and any report (an
out-of-bounds access, a signed overflow, an invalid enum load, a misaligned access)
fails the run.  No GPU is used: the calls that get past validation report the HIP
error of a machine without a device.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from exact_attention_62_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime_or_skip() -> str:
    try:
        return B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))


def test_abi_and_schedule_suites_under_asan_and_ubsan(tmp_path):
    runtime = _runtime_or_skip()
    lib = B.build(out=str(tmp_path / "libfa2_san.so"), sanitize=True)
    log = str(tmp_path / "san")
    env = dict(os.environ,
               FA2_LIBRARY=lib,
               LD_PRELOAD=runtime,
               # Python itself is not instrumented and keeps objects alive at exit.
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_abi.py", "tests/test_schedule.py"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=900)
    reports = "".join(open(p).read() for p in sorted(glob.glob(log + ".*")))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + "\n" + reports[:6000])
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


def test_sanitizer_flags_stay_host_only():
    """Every -fsanitize= of the build sits directly after -Xarch_host: device code is
    never built with a sanitizer."""
    for flags in (B.SANITIZE_FLAGS,):
        for i, f in enumerate(flags):
            if f.startswith("-fsanitize"):
                assert i > 0 and flags[i - 1] == "-Xarch_host", flags
