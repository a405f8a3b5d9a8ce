"""The library's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the same sources with the sanitizers on the host side only (the gfx950
device code is built as usual and never runs here), then runs the host-only
pool and engine tests against that build in a child process.  A heap
overflow, use after free or undefined operation in the allocator, page
tables, plans or engine aborts the child, which fails this test.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from heterogeneous_adapter_gemm_amd import build as B

OUT = os.path.join(B.BUILD_DIR, "host_sanitizers")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build() -> str:
    os.makedirs(OUT, exist_ok=True)

    def one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([B.HIPCC, *B.FLAGS, *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(len(B.SOURCES)) as ex:
        objs = list(ex.map(one, B.SOURCES))
    lib = os.path.join(OUT, "libhagemm.so")
    r = subprocess.run([B.HIPCC, "-shared", f"--offload-arch={B.ARCH}", *objs, "-fsanitize=address,undefined",
                        "-shared-libsan", "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


@pytest.mark.timeout(900)
def test_host_logic_under_address_and_ub_sanitizers():
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    lib = _build()
    env = dict(os.environ, HAGEMM_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_pool_host.py", "tests/test_engine_host.py"],
                       cwd=root, env=env, capture_output=True, text=True)
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
