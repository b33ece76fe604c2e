"""The host plan code (validation, table images, plan cache) built with the
host compiler under AddressSanitizer and UndefinedBehaviorSanitizer and run
against a fake device whose memory is host memory (tests/native/plan_check.cpp).
No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "optimizer_muon_step_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_plan_code_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", ROCM_INC, "-I", CSRC, os.path.join(CSRC, "plan_host.cpp"),
           os.path.join(ROOT, "tests", "native", "plan_check.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
