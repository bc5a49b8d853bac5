"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds the host-sanitized library (unified_block_sparse_amd.sanitize_build) and runs
tests/test_abi.py against it in a child process with the ASan runtime preloaded. Any
sanitizer report aborts that process (UBSan without recovery), so the run must pass
and print none."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_suite_clean_under_asan_and_ubsan():
    from unified_block_sparse_amd import sanitize_build
    lib = sanitize_build.build()
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "the library is not instrumented"
    env = dict(os.environ)
    env.update(UBS_LIBRARY=lib, LD_PRELOAD=sanitize_build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = ("import sys, pytest, unified_block_sparse_amd as u; "
            f"assert u.LIB_PATH == {lib!r}, u.LIB_PATH; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
