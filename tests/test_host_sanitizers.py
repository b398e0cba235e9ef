"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of libspecverify.so whose host code (argument validation,
workspace-size arithmetic, status strings) is instrumented, with
``-Xarch_host`` before every sanitizer flag so that no device code is, and
runs the ABI tests against it in a child process with the sanitizer runtime
preloaded and every report fatal.  The ABI tests make no HIP call that reaches
the GPU: every call they make returns before its launch.
"""
import os
import subprocess
import sys
import tempfile

import pytest

from sampling_spec_verify_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run([B.HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_tests_pass_under_host_sanitizers():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not found")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "libspecverify_san.so")
        flags = [f for f in B.FLAGS if f != "-O3"] + [
            "-O1", "-g",
            "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
        ]
        srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
        r = subprocess.run([B.HIPCC, *flags, "-I", B.INCLUDE, "-I", B.CSRC, *srcs, "-o", lib],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        env = dict(os.environ, SPECVERIFY_LIB=lib, LD_PRELOAD=runtime,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                            "-x", "-q", "-s", "-p", "no:cacheprovider"],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
        assert " passed" in out
