"""The host library's integer work under AddressSanitizer and
UndefinedBehaviorSanitizer: mlora_host.cpp is compiled with g++ together with
a driver (host_sanitize.cpp) that calls every host entry point on edge cases
and a seeded fuzz; any sanitizer report or failed check fails the test. No
GPU code is built or run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "moe_expert_lora_amd", "csrc"),
           os.path.join(HERE, "host_sanitize.cpp"),
           os.path.join(ROOT, "moe_expert_lora_amd", "csrc", "mlora_host.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "clean" in run.stdout
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr
