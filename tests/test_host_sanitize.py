"""The C-ABI host layer (csrc/fkl_api.cpp: argument checks, workspace and
pass planning) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, without HIP, and driven over edge and random
shapes by tests/host_sanitize/plan_check.cpp, whose stub launchers check every
workspace region and operand-view limit the kernels rely on (no GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


def test_host_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the ROCm headers")
    exe = tmp_path / "plan_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "output_projection_kl_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_sanitize", "plan_check.cpp"),
           os.path.join(ROOT, "output_projection_kl_amd", "csrc", "fkl_api.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("FKL_VALIDATE", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "OK" in r.stdout and "failures 0" in r.stdout
