"""The library's host logic (problem and schedule checks, lane layouts,
workspace layout, candidate lists, cost model, format plan, signature, cache
log lines) built with g++ under the address and undefined-behaviour
sanitizers and driven by seeded random problems, schedules and corrupted
cache lines (host_fuzz.cpp states the invariants it checks).  No GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_logic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "csr_sparse_attention_amd", "csrc", "host.cpp"),
           os.path.join(ROOT, "tests", "host_fuzz.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures 0" in r.stdout
