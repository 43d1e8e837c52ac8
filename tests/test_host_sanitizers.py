"""The host code of the library (argument checks, split planning, workspace
sizing, the C-ABI entry points' error paths) under AddressSanitizer and
UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on the host pass of every source
(device code as usual) into _build/sanitize/, then test_abi.py and
test_bench_host.py run in a child Python process that loads that build
(DDTREE_LIBRARY) with the clang sanitizer runtime preloaded.  Any report makes
the child abort (halt_on_error, no recovery), so the run must end cleanly and
print none.  No GPU is used.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_bench_host_tests_clean_under_asan_ubsan():
    from tree_verification_build_amd import _build
    try:
        hipcc = _build._hipcc()
        runtime = _build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    assert shutil.which(hipcc) or os.path.exists(hipcc)
    lib = _build.build(sanitize=True)
    env = dict(os.environ, DDTREE_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_bench_host.py",
           "-m", "not gpu", "-q", "-x", "-s", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("runtime error", "AddressSanitizer", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
    assert " passed" in out
