"""Build libdsa.so (HIP, gfx950) in-tree with hipcc.

    python -m long_context_sparse_index_amd.build

Compiles every csrc/*.hip to an object under _build/ and links the shared
library next to this file.  Always recompiles (the build is the check that
the sources compile for gfx950).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Host AddressSanitizer build of the C-ABI shim (host code only; device code is
# built as usual): objects and library under _build/host_asan/.
HOST_ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-Xarch_host", "-g"]
ASAN_BUILD = os.path.join(BUILD, "host_asan")
ASAN_LIB = os.path.join(ASAN_BUILD, "libdsa_host_asan.so")


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to LD_PRELOAD into a
    host process that loads the host-ASan library), or '' if absent."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm", "lib", "clang")
    for lib in sorted(glob.glob(os.path.join(root, "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))):
        return lib
    return ""


def _compile(src: str, out_dir: str = None, extra=()) -> str:
    obj = os.path.join(out_dir or BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def build_host_asan(verbose: bool = True) -> str:
    """The library with AddressSanitizer on its host code (for host-side tests of
    the C ABI on a machine without a GPU)."""
    os.makedirs(ASAN_BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, ASAN_BUILD, HOST_ASAN_FLAGS), srcs))
    rt = asan_runtime()
    if not rt:
        raise RuntimeError("no AddressSanitizer runtime found next to the compiler")
    # the instrumented objects link against the shared sanitizer runtime itself
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", ASAN_LIB, *objs, rt]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(f"built {ASAN_LIB} (host AddressSanitizer)")
    return ASAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--host-asan":
        build_host_asan()
    else:
        build()
