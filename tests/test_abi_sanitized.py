"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (argument checks, partition planning, workspace sizing, struct tables) is built with g++
and both sanitizers, the device launchers replaced by stubs (csrc/host_stubs.cpp), and the whole
host-side ABI test files (the checks and the argument fuzzing) run against it in a child process with the sanitizer runtime preloaded:
any out-of-bounds access, use after free or undefined behaviour in that code fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    try:
        r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    except OSError:
        return None
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_under_address_and_undefined_behaviour_sanitizers():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from two_tower_cross_amd import build
    lib = build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=asan, TWOTOWER_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_abi_fuzz.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
