"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: hcr_api.cpp (every argument
check of include/hcr.h) is built with the host compiler and -fsanitize=address,undefined, with host-only
stand-ins for the kernel launchers (tests/asan/host_stubs.cpp), and tests/test_abi.py and
tests/test_abi_contract.py run against that build in a child process with the sanitizer runtime preloaded.
No GPU is used: those tests make only calls the checks reject."""

import os
import shutil
import subprocess
import sys

import pytest

from tests.libhcr_util import ROOT

CSRC = os.path.join(ROOT, "bf16_hyper_connection_amd", "csrc")


def _cxx():
    for c in ("g++", "c++"):
        if shutil.which(c):
            return c
    return None


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    cxx = _cxx()
    if cxx is None:
        pytest.skip("no host C++ compiler")
    out = str(tmp_path_factory.mktemp("asan") / "libhcr_asan.so")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "hcr_api.cpp"), os.path.join(ROOT, "tests", "asan", "host_stubs.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    libasan = subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(libasan) and os.path.exists(libasan), libasan
    return out, libasan


def test_abi_checks_clean_under_asan_and_ubsan(asan_lib):
    lib, libasan = asan_lib
    env = dict(os.environ, HCR_LIB=lib, LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_abi_contract.py",
                        "-k", "not source_hash"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
