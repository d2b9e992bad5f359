"""The library's host code under AddressSanitizer and UBSan (CPU only).

The C-ABI layer (argument checks, size arithmetic, error reporting, the block
manager) is host code. This test builds the library from the same sources with
build.py's flags plus AddressSanitizer and UndefinedBehaviorSanitizer (no
recovery) on the host pass only (the device code
is built as always), then runs tests/test_abi.py against that build in a
child process with the sanitizer runtime preloaded: every entry point's
refusal paths run under them, and any memory error or undefined behaviour
aborts the child.
"""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_151_amd")


def _build_module():
    # loaded by path: importing the package itself needs the built library
    spec = importlib.util.spec_from_file_location("pa_build_flags", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_refusals_under_host_address_sanitizer(tmp_path):
    b = _build_module()
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("the clang AddressSanitizer runtime was not found")
    lib = tmp_path / "libpa_host_asan.so"
    cmd = [hipcc, *b.HIP_FLAGS, "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host",
           "-fno-sanitize-recover=all", "-Xarch_host",
           "-fno-omit-frame-pointer", "-shared-libsan", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), *b.sources(), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, PA_ABI_LIB=str(lib), LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider"], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, (r.stdout[-3000:] +
                                                                      r.stderr[-3000:])
    assert " passed" in r.stdout, r.stdout[-3000:]
