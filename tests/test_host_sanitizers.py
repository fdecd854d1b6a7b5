"""The host core (quantizer tables, codebook set-up and teardown, argument
validation of every entry point) built as plain C++ with AddressSanitizer
and UndefinedBehaviorSanitizer against host stand-ins for the HIP runtime
and the kernel launchers (tests/host_sanitize/stubs.cpp), run on the CPU.
Any heap error, leak or undefined behaviour fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CXX = shutil.which("amdclang++") or "/opt/rocm/bin/amdclang++"


@pytest.mark.skipif(not os.path.exists(CXX), reason="no clang++ for the host build")
def test_host_core_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_check")
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "kv_cache_vector_rotate_amd", "csrc", "tq_host.cpp"),
           os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "host_check.cpp"), "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-6000:]
    assert "validation: ok" in run.stdout
