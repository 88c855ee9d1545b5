"""The C++ block manager under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, built with g++): tests/bm_fuzz.cpp drives seeded streams of
valid and invalid calls and checks the manager's invariants after each."""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fuzz_binary():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = os.path.join(tempfile.mkdtemp(prefix="pkv_bm_fuzz_"), "bm_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           f"-I{ROOT}/include", f"-I{ROOT}/paged_kv_cache_325_amd/csrc",
           os.path.join(ROOT, "tests", "bm_fuzz.cpp"),
           os.path.join(ROOT, "paged_kv_cache_325_amd", "csrc", "block_manager.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return out


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6])
def test_block_manager_under_sanitizers(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_binary, str(seed), "4000"], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 check failures" in r.stdout
