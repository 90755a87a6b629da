"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: kvsel_api.cpp built with g++ and the sanitizers, linked with
host-only stand-ins for the GPU side (tests/host_asan/launch_stubs.cpp: a
gfx950 device, and launches that check every array a kernel would touch
against the caller's buffers), driven through every entry point by
tests/host_asan/abi_driver.cpp: invalid problems and arguments, and valid
problems from one key to 2^20 keys, whole-prefix, fused and unfused,
streaming, warm-up and budgets."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_asan")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "attention_token_selection_amd", "csrc"),
           "-I" + HERE, os.path.join(ROOT, "attention_token_selection_amd", "csrc", "kvsel_api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("KVSEL_UNFUSED", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "0 checks failed, 0 launch checks failed" in out, out[-2000:]
