"""The CPU ABI tests again, against a host build of the C ABI instrumented
with AddressSanitizer and UndefinedBehaviorSanitizer (argument validation,
overlap and stride arithmetic, size helpers).  Any sanitizer report aborts the
child run and fails this test.  Skipped where the ASan runtime is missing, or
where the process environment already preloads a library (the sanitizer
runtime has to come first, and this test does not replace another preload)."""

import os
import subprocess
import sys

import pytest

from differential_attention_forward_amd.build import asan_runtime, build_sanitized_host

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_cpu_under_sanitizers():
    rt = asan_runtime()
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not found")
    if os.environ.get("LD_PRELOAD") or os.path.exists("/etc/ld.so.preload"):
        pytest.skip("a library is already preloaded in this environment")
    lib = build_sanitized_host(os.path.join(ROOT, "_build", "san"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ, DIFFATTN_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "passed" in res.stdout
