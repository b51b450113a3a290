"""The host side of the C ABI (argument checks, plans, workspace sizes, the
plan override, the static-scratch refusals) under AddressSanitizer: the
library is rebuilt with the host code instrumented (the device code as
usual), and test_abi_host.py runs against it in a child process with the
sanitizer runtime preloaded.  CPU only."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp4_kv_cache_indexer_amd import build as B

HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    clang = os.path.join(os.path.dirname(B.HIPCC), "..", "llvm", "bin", "clang")
    try:
        rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                            text=True, timeout=60).stdout.strip()
    except OSError:
        return None
    return rt if os.path.isabs(rt) and os.path.exists(rt) else None


def _build_asan_library():
    out = os.path.join(B.BUILD, "asan")
    os.makedirs(out, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        r = subprocess.run([B.HIPCC, *B.CFLAGS, *HOST_ASAN, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, B.sources()))
    lib = os.path.join(out, "libcsa2_asan.so")
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_ASAN, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


def test_abi_host_under_address_sanitizer():
    if not os.path.exists(B.HIPCC):
        pytest.skip("no hipcc")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime")
    lib = _build_asan_library()
    env = dict(os.environ, CSA2_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    # the child maps the instrumented build, with the sanitizer runtime live
    probe = ("import ctypes; from fp4_kv_cache_indexer_amd import csa2 as C; C.lib(); "
             "m = open('/proc/self/maps').read(); "
             "print('asan-lib' if 'libcsa2_asan.so' in m else 'other-lib', "
             "hasattr(ctypes.CDLL(None), '__asan_init'))")
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=300,
                       cwd=B.ROOT)
    assert r.stdout.split() == ["asan-lib", "True"], r.stdout + r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(B.ROOT, "tests", "test_abi_host.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=B.ROOT)
    log = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in log, log[-6000:]
    assert r.returncode == 0, log[-6000:]
    assert " passed" in r.stdout
