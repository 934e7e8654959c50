"""The library's host-side C ABI (host.cpp: best-first tree builder, tree
validator, status strings, contract errors) under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/sanitize/host_abi_sanitize.cpp is compiled together with host.cpp by the
host compiler (g++, no GPU code involved) with -fsanitize=address,undefined and
run: 2000 random candidate tables plus the contract's error cases. Any
sanitizer report or failed property check fails the test. No GPU is needed.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the ROCm headers")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "draft_tree_verification_dt_amd", "csrc"),
           os.path.join(ROOT, "draft_tree_verification_dt_amd", "csrc", "host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_abi_sanitize.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"sanitizer build failed:\n{r.stderr}"


def test_host_abi_under_address_and_undefined_behavior_sanitizers(tmp_path):
    exe = str(tmp_path / "host_abi_sanitize")
    _build(exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if r.returncode != 0 and "LeakSanitizer has encountered a fatal error" in r.stderr:
        # leak checking cannot run under some tracers; the rest of ASan still can
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "host ABI checks passed" in r.stdout, report
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, report
