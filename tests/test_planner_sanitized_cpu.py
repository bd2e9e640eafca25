"""The host plan rule under address and undefined-behaviour sanitizers.

tests/planner_fuzz.cpp is built with g++ together with the library's planner source
(csrc/planner.cpp, a plain C++17 file with no HIP dependency) and run on a few
thousand random plans: ragged length mixes with empty requests, lengths up to 2e7
tokens (every digit of the radix ordering), page sizes 1-256, sliding windows, random
schedules and the cascade's every-group-merges mode. The driver checks every item
against its request and that every partial-state slot is written exactly once; the
sanitizers check the rule's memory accesses and integer arithmetic. Skipped when no
g++ is on PATH.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_cache_173_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_rule_under_sanitizers(tmp_path):
    exe = str(tmp_path / "planner_fuzz")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-I", CSRC, os.path.join(HERE, "planner_fuzz.cpp"),
         os.path.join(CSRC, "planner.cpp"), "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "failures 0" in run.stdout, run.stdout
