"""The C ABI's host-side argument checks under AddressSanitizer (CPU only).

api.cpp is compiled with the sanitizer on its host code only (the device
pass is untouched) and linked with tests/asan_launch_stubs.cpp, which stands
in for the kernel launchers and the dispatch table.  The ABI validation tests
of tests/test_abi.py then run in a child process against that library, with
the sanitizer's runtime preloaded: every refused argument set, every empty
problem and every accepted one walks api.cpp's checks with instrumented
loads and stores.  The tests that read the real dispatch table are left out
(the stand-in has one fixed tile).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scaled_dot_product_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _runtime():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        return None
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-2000:] + r.stderr[-4000:]


def _build(tmp):
    api_o = os.path.join(tmp, "api.o")
    stubs_o = os.path.join(tmp, "stubs.o")
    lib = os.path.join(tmp, "libsdpa03_asan.so")
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    _run([CLANG, "-O1", "-g", "-fPIC", "-std=c++17", "-fsanitize=address",
          "-fno-omit-frame-pointer", "-I", CSRC, "-c",
          os.path.join(ROOT, "tests", "asan_launch_stubs.cpp"), "-o", stubs_o])
    _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-Xarch_host", "-fsanitize=address",
          "-shared-libsan", api_o, stubs_o, "-o", lib])
    return lib


def test_abi_validation_under_address_sanitizer(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("hipcc or the AddressSanitizer runtime is not installed")
    lib = _build(str(tmp_path))
    syms = subprocess.run(["nm", "-u", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__asan_report_store" in syms, "not instrumented"
    env = dict(os.environ, SDPA03_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0:exitcode=86")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
         "-p", "no:cacheprovider", "-k",
         "not kernel_config and not splitk_plan and not scratch_limit"],
        capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]
    shutil.rmtree(str(tmp_path), ignore_errors=True)
