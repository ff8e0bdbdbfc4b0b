"""The host pool code built alone with AddressSanitizer and UBSan (g++, no
HIP), driven by a randomized stress that checks the pool's invariants."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pool_stress_under_asan_ubsan(tmp_path):
    exe = tmp_path / "pool_stress"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "native", "pool_stress.cpp"),
           os.path.join(ROOT, "paged_kv_cache_218_amd", "csrc", "pool.cpp"),
           os.path.join(ROOT, "paged_kv_cache_218_amd", "csrc", "prefix_cache.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # the environment is passed on as it is; ASan is told not to insist on
    # being the first library loaded
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "pool stress ok" in r.stdout
