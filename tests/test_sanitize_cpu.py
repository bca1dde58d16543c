"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the C-ABI
layer (kda_api.cpp as plain host C++, kernel launchers stubbed out) and of
the fp64 C oracle, through tests/sanitize/host_driver.cpp.  CPU only: no
GPU code is built with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None
                    or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
                    reason="needs g++, gcc and the ROCm headers")
def test_host_layers_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g", "-O1"]
    obj = tmp_path / "oracle.o"
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-c", os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    "-o", str(obj)] + san, check=True)
    exe = tmp_path / "host_driver"
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "gated_delta_rule_95_amd", "csrc"),
           os.path.join(ROOT, "gated_delta_rule_95_amd", "csrc", "kda_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), str(obj),
           "-o", str(exe), "-fopenmp", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"] + san
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized host checks passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
