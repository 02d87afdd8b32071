"""The library's host code (rate tables, codebooks, rate allocation, head layouts, plan
construction, the decode kernel's K-block slot order) built with AddressSanitizer and
UndefinedBehaviorSanitizer into the property harness tests/host_sanitize.cpp and run over
several seeds. Host compiler only: no GPU code is built or run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    cxx = CLANG if os.path.exists(CLANG) else shutil.which("clang++")
    if cxx is None:
        pytest.skip("no clang++ with the sanitizer runtimes")
    exe = str(tmp_path_factory.mktemp("hs") / "host_sanitize")
    csrc = os.path.join(ROOT, "packed_cache_attention_tq_amd", "csrc")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "host_sanitize.cpp"), os.path.join(csrc, "gtq_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_under_sanitizers(harness, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([harness, "150", str(seed)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout
