"""The C ABI's argument validation built host-only with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer, with every error path forced by a C++ driver
(capi_validation_driver.cpp): each call must return its documented status before
reaching a launcher (the launchers are stubs that abort), with no sanitizer report.
The driver also stands in for the HIP runtime calls the C ABI makes, so a failing
decode-workspace allocation (FA_ERR_NOMEM, nothing launched) is forced on the CPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_validation_paths_under_sanitizers(tmp_path):
    exe = tmp_path / "capi_validation"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "exact_io_aware_74_amd", "csrc"),
           os.path.join(HERE, "capi_validation_driver.cpp"),
           os.path.join(ROOT, "exact_io_aware_74_amd", "csrc", "fa_capi.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr
    assert "all validation paths returned the expected status" in run.stdout
