"""The C-ABI shim's host code under AddressSanitizer: the host-side ABI tests
(argument checks, workspace sizes, the IndexShare schedule, the no-device path)
run against a build whose host code is instrumented, in a child process with
the sanitizer runtime preloaded.  Any invalid host memory access in the shim
aborts the child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

from long_context_sparse_index_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from long_context_sparse_index_amd import dsa
dsa._LIB_PATH = {lib!r}
import ctypes
L = dsa.lib()
assert ctypes.CDLL(None).__getitem__("__asan_init")  # the runtime is in the process
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", {test!r}]))
"""


def test_abi_host_tests_under_host_asan():
    rt = build.asan_runtime()
    if not rt:
        pytest.skip("no AddressSanitizer runtime next to the compiler")
    lib = build.build_host_asan(verbose=False)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    code = CHILD.format(root=ROOT, lib=lib, test=os.path.join(ROOT, "tests", "test_abi_host.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout
