"""The library's host bookkeeping (pool.hip: create, slab append over one or
several launches, the roll-back of a failed append, the host table mirror
against the device tables, argument errors, storage identities) built with
the host compiler under AddressSanitizer, UndefinedBehaviorSanitizer and
LeakSanitizer, against a stand-in runtime whose launches do their table
writes and zero fills on host memory (tests/host_asan).  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_bookkeeping_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_asan")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined",
           "-I", os.path.join(HERE, "stub"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "decode_memory_amd", "csrc"),
           "-x", "c++", os.path.join(ROOT, "decode_memory_amd", "csrc", "pool.hip"),
           "-x", "c++", os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host bookkeeping ok" in r.stdout
