"""The C ABI's host code (argument checks, workspace sizing, launch plan)
built with the address and undefined-behaviour sanitizers and driven through
every accepted and rejected argument pattern, with stub launchers in place of
the GPU kernels (tests/abi_host_check.cpp).  Host compiler only: no device
code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mla_attention_fp8_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host C++ compiler")
def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "0 failed" in r.stdout
