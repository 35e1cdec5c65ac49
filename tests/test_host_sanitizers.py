"""The host planner and the address walk (csrc/mk_plan.cpp, csrc/mk_check.cpp)
built with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code
only) and run over the tiny, Llama-1B, long-context and Llama-8B plans: no
sanitizer report, every walk clean."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "persistent_megakernel_cu_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_and_walk_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "walk")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "host_walk_driver.cpp"), os.path.join(CSRC, "mk_check.cpp"),
           os.path.join(CSRC, "mk_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 4 and all("violations=0" in line for line in lines), r.stdout
