"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds ``tests/host_check/abi_host_check.cpp`` with the library's host sources
(argument checks, launch plans, workspace carving, cap policy) using g++, with
the kernel launches replaced by recorders (no GPU, no device memory), and runs
it: every accepted call must carve its workspace inside the caller's buffer,
every rejected call must leave a message, and the sanitizers must stay quiet.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verify_dspk_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_host_check"
    srcs = [os.path.join(ROOT, "tests", "host_check", "abi_host_check.cpp")] + \
        [os.path.join(CSRC, f) for f in ("api.cpp", "plan.cpp", "policy.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC] + srcs + ["-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host check ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
