"""The host tests of the K/V allocator and the scheduler, run against the
host-only part of the library built with AddressSanitizer and
UndefinedBehaviorSanitizer (any heap error, out-of-bounds access or
undefined behaviour in kv.cpp, sched.cpp or status.cpp aborts the run).
CPU only: the sanitized build holds no GPU code."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_tests_under_asan_and_ubsan():
    from orca_selective_iteration_amd.build import build_host_sanitized
    lib = build_host_sanitized()
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("no AddressSanitizer runtime for g++")
    env = dict(os.environ, ORCA_LIB=lib, ORCA_HOST_ONLY="1", LD_PRELOAD=asan,
               # the interpreter's own allocations are not under test
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi_host.py"),
         "-k", "allocator or scheduler"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
