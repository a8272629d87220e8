"""The library's host-only C++ (block allocator, argument checks, RoPE table,
work-partition replay) under AddressSanitizer, UndefinedBehaviorSanitizer and
LeakSanitizer, on the CPU.

The host-only sources build with g++ (no HIP) into a sanitizer-instrumented
library.  Two runs use it, and any sanitizer report fails them:

* a C++ driver (``host_sanitize_driver.cpp``) calls every host-only entry
  point over seeded random inputs, valid and invalid, with leak checks on;
* the ABI and allocator tests run against that library in a child Python
  with the ASan runtime preloaded (leak checks off there: the interpreter
  keeps memory of its own until exit); the tests that need entry points only
  the full HIP library exports are skipped in that run.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_decode_step_amd", "csrc")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("host_api.cpp", "block_alloc.cpp")]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]
COMMON = ["-std=c++17", "-O1", "-g", "-ffp-contract=off",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def gxx(args, cwd):
    res = subprocess.run(["g++", *COMMON, *SANITIZE, *args], capture_output=True, text=True,
                         cwd=cwd)
    assert res.returncode == 0, res.stdout + res.stderr


@pytest.fixture(scope="module")
def host_build(tmp_path_factory):
    d = tmp_path_factory.mktemp("hostsan")
    lib = str(d / "libpkv_host_sanitized.so")
    gxx(["-shared", "-fPIC", *HOST_SOURCES, "-o", lib], d)
    drv = str(d / "host_sanitize_driver")
    gxx([os.path.join(HERE, "host_sanitize_driver.cpp"), *HOST_SOURCES, "-o", drv], d)
    return lib, drv


def sanitizer_env(**extra):
    env = dict(os.environ)
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_driver_is_clean_under_asan_ubsan_lsan(host_build):
    _, drv = host_build
    res = subprocess.run([drv], capture_output=True, text=True, timeout=600,
                         env=sanitizer_env(ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "host entry points clean" in res.stdout
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr


def test_abi_and_allocator_tests_pass_against_the_sanitized_library(host_build):
    lib, _ = host_build
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), "gcc's ASan runtime not found"
    env = sanitizer_env(PKV_HOST_LIBRARY=lib, LD_PRELOAD=asan,
                        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         os.path.join(HERE, "test_abi.py"), os.path.join(HERE, "test_block_alloc.py")],
        capture_output=True, text=True, timeout=900, cwd=ROOT, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in res.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out
