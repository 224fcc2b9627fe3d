"""The library's host-side planning code (block_sparse_attention_40_amd/csrc/
moba_plan.cpp: argument validation and workspace layouts of the forward, the
forward with a given workspace, the backward and decode) built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, no GPU code) and run
over a sweep of shapes that includes the overflow edges of its size
arithmetic (tests/host/plan_sweep.cpp): every accepted plan must be
self-consistent, and no sanitizer may fire."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_plan_sweep_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "plan_sweep")
    build = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-o", exe, os.path.join(ROOT, "tests", "host", "plan_sweep.cpp"),
             os.path.join(ROOT, "block_sparse_attention_40_amd", "csrc", "moba_plan.cpp")]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr, r.stderr[-4000:]
    print(r.stdout.strip())
