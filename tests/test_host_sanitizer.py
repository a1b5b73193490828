"""The C ABI's host code -- argument validation, workspace sizing, launch
planning -- under AddressSanitizer and UndefinedBehaviorSanitizer: the ABI
test suite runs in a child process against libkvsel_hostcheck.so (api.cpp
built with g++ -fsanitize=address,undefined, every kernel launch replaced by
a check of its launch description), with the ASan runtime preloaded.  Any
sanitizer report, or a launch description that fails its check, aborts the
child and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "token_selection_tsp_amd", "libkvsel_hostcheck.so")


def _asan_runtime():
    try:
        out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_abi_suite_under_asan_ubsan():
    if not os.path.exists(LIB):
        from token_selection_tsp_amd import build as _b
        _b.build_hostcheck()
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("no ASan runtime (gcc) on this host")
    # the library really is instrumented: it calls into both runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True,
                          check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, KVSEL_TEST_LIB=LIB, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
