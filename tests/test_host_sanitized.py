"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

The library is rebuilt with its host code instrumented (argument checks,
code-book and bucket-table derivation, launch planning; the device code is
unchanged) and the host-only ABI tests run against that build in a fresh
interpreter with the sanitizer runtime preloaded.  Any invalid access or
undefined behaviour aborts that interpreter, so the run must pass as it does
against the regular build."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    if not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")):
        pytest.skip("hipcc is not available")
    from dequant_matmul_nf4_amd import build
    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=build.sanitizer_runtime(), NF4_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    return env, lib


def test_sanitized_build_is_instrumented(san_env):
    _, lib = san_env
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_" in out
    assert "__ubsan_handle_" in out


def test_host_abi_tests_pass_under_the_sanitizers(san_env):
    env, _ = san_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


def test_sanitizer_runtime_catches_an_overflow(san_env):
    """The preloaded runtime is live: the code book written into a 32-byte
    heap buffer (it needs 64) is reported as a heap overflow."""
    env, _ = san_env
    code = ("import ctypes, dequant_matmul_nf4_amd as nf4\n"
            "libc = ctypes.CDLL(None); libc.malloc.restype = ctypes.c_void_p\n"
            "p = libc.malloc(32)\n"
            "nf4.lib().nf4_codebook(ctypes.cast(p, ctypes.POINTER(ctypes.c_float)))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
