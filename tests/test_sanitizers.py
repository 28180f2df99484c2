"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

libpxa_san.so is the library built with both sanitizers on its host code
(block_sparse_long_proxy_amd/build.py --sanitize); the host-side tests of the
validation paths, workspace sizing and layouts (tests/test_abi_host.py) run
against it in a child process with the ASan runtime preloaded.  Any
sanitizer report aborts that process and fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
from block_sparse_long_proxy_amd import _binding as B
B.load_library(sys.argv[2])
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", sys.argv[3]]))
"""


def test_abi_host_tests_pass_under_asan_and_ubsan():
    from block_sparse_long_proxy_amd import build
    try:
        lib = build.build(sanitize=True)
        runtime = build.asan_runtime()
    except RuntimeError as e:           # no ROCm toolchain on this machine
        pytest.skip(str(e))
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm and "__ubsan_handle" in nm, "library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, lib,
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in out, out
