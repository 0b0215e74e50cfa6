"""The C-ABI validation of libfp4idx (pack_token_amd/csrc/fp4idx_api.cpp)
built for the host with AddressSanitizer and UndefinedBehaviorSanitizer, the
kernel launchers replaced by recorders (tests/native/api_host_stubs.cpp), and
driven by tests/native/api_sanitize_driver.cpp: extreme sizes must be refused
without overflow, valid calls must hand the launchers the expected
descriptors, and a failed launch must surface as FP4IDX_EHIP.  CPU only."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validation_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "driver")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(ROOT, "pack_token_amd", "csrc"), "-I", NATIVE,
               os.path.join(ROOT, "pack_token_amd", "csrc", "fp4idx_api.cpp"),
               os.path.join(NATIVE, "api_host_stubs.cpp"),
               os.path.join(NATIVE, "api_sanitize_driver.cpp"), "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        # verify_asan_link_order=0: the runtime need not be first in the library list
        env = dict(os.environ,
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
