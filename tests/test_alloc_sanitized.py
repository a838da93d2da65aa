"""Build the host allocator with -fsanitize=address,undefined (g++, host code
only) and run a random-operation stress through its C ABI."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_411_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_allocator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "alloc_stress")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "alloc_stress.cpp"),
           os.path.join(CSRC, "block_allocator.cpp"), os.path.join(CSRC, "status.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # the environment is passed on unchanged; ASan is told not to insist on
    # being first in the library list
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
