"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

A host-only build of libpred (argument checks, sizing, the projection generator
and launch set-up; no device code) runs tests/test_abi.py in a child process
with the sanitizer runtime preloaded.  Any sanitizer report fails the test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded here; the sanitizer runtime would replace it")
    from rank_kv_block_amd import build
    lib = build.build_host_sanitized()
    runtime = build.sanitizer_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    env = dict(os.environ, LD_PRELOAD=runtime, PRED_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    # the runtime really is in the child (a silent no-op preload would pass everything)
    probe = subprocess.run([sys.executable, "-c", "print('libclang_rt.asan' in open('/proc/self/maps').read())"],
                           env=env, capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip() == "True", probe.stdout + probe.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
