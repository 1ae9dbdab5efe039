"""The library's host-only logic under address and undefined-behaviour
sanitizers (no GPU).

``sparse_attention_kv_request_amd/csrc/host_logic.h`` holds everything the C
ABI computes on the host without a HIP call: configuration derivation and
limits, the encoding of an imported cache instance (key->slot table, LRU
order, CLOCK reference bitmap) and the decoding of an export, and the
bookkeeping of the timing events (whole triples per call on every return
path).  ``tests/host_logic_check.cpp`` drives it with table cases, random
and extreme values; this test builds that driver with g++ and the
sanitizers and runs it.
"""
import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_logic_under_sanitizers(tmp_path):
    exe = tmp_path / "host_logic_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{ROOT / 'include'}", f"-I{ROOT / 'sparse_attention_kv_request_amd' / 'csrc'}",
           str(ROOT / "tests" / "host_logic_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all" in res.stdout and "checks passed" in res.stdout, res.stdout
