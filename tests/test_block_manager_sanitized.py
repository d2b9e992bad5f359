"""The native host block manager under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

csrc/block_manager.cpp is host C++ with no GPU code, so it can be built with
g++ and both sanitizers, without the rest of the library. tests/bm_sanitize.cpp
drives its C ABI through seeded random operation sequences and the calls the
header defines as errors, and checks the manager's state after every operation
(reference counts against the live tables, free count, table lengths, slots,
copy pairs, partial application of a failed append). Any memory error or
undefined behaviour aborts the run; any failed check fails it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_151_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"   # pa.h names hipStream_t (the host API header only)


def test_block_manager_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(HIP_INCLUDE):
        pytest.skip("g++ or the HIP headers not found")
    exe = tmp_path / "bm_sanitize"
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", HIP_INCLUDE,
             "-I", CSRC, os.path.join(ROOT, "tests", "bm_sanitize.cpp"),
             os.path.join(CSRC, "block_manager.cpp"), "-o", str(exe)]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "40"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "bm_sanitize: ok" in r.stdout, r.stdout + r.stderr[-4000:]
