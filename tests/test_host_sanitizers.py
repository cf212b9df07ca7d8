"""Host-only sanitizer build of the library's validation and launch planning.

decode_attention_mfa_amd/csrc/host_plan.cpp holds every host rule of the
decode entry points (descriptor and pointer validation, the split heuristic,
the workspace layout) and uses no HIP, so it is compiled here with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer together with
tests/host/plan_sweep.cpp, which drives it over a grid of edge values and
checks the plan's invariants.  Any out-of-bounds access, signed overflow or
other undefined behaviour aborts the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_mfa_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_plan_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "plan_sweep"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "plan_sweep.cpp"),
           os.path.join(CSRC, "host_plan.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "failures 0" in run.stdout
