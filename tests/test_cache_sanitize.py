"""The expert slot cache's host code (expert_cache.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer by g++ (host code only, no HIP) and driven through random
routing streams (tests/cache_sanitize.cpp): no memory error, no undefined behaviour, and
the slot invariants hold after every call. No GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_expert_matmul_k3moe_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_cache_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "cache_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", CSRC,
           os.path.join(ROOT, "tests", "cache_sanitize.cpp"),
           os.path.join(CSRC, "expert_cache.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # other preloaded libraries may precede the ASan runtime: do not insist on its order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout}\n{r.stderr}"
    assert "ok" in r.stdout
