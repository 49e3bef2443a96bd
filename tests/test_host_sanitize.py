"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, no GPU:

- the fp64 oracle (oracle/k3oracle.c), built by gcc with both sanitizers into a driver
  (tests/host_sanitize_oracle.c) that runs small layers of several shapes through every
  exported routine and checks their invariants;
- the C ABI's host code (argument validation, workspace layout and the slot plan in
  k3moe_api.cpp and expert_cache.cpp), built by hipcc with the sanitizers on the host side
  only and linked with the kernels' objects into a library that a sanitized driver
  (tests/host_sanitize_api.cpp) calls with invalid arguments, T = 0, sizing and cache plans,
  none of which reaches a HIP call.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_expert_matmul_k3moe_amd", "csrc")
INC = os.path.join(ROOT, "include")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nrc={r.returncode}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
          "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "tests", "host_sanitize_oracle.c"),
          os.path.join(ROOT, "oracle", "k3oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert "ok" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_abi_host_code_under_sanitizers(tmp_path):
    from mxfp4_expert_matmul_k3moe_amd import build as lib_build
    hip_flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                 "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
                 "-packed-fp32-ops", "-I", CSRC, "-I", INC]
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

    def comp(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = ["hipcc", *hip_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):  # the host code under test
            cmd[1:1] = ["-x", "hip"]
            cmd += san_host
        _run(cmd)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, lib_build.SOURCES))
    lib = str(tmp_path / "libk3moe_san.so")
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs])
    clang = shutil.which("amdclang++") or "/opt/rocm/llvm/bin/clang++"
    exe = str(tmp_path / "abi_san")
    _run([clang, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", INC,
          os.path.join(ROOT, "tests", "host_sanitize_api.cpp"), lib,
          "-Wl,-rpath," + str(tmp_path), "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "ok" in r.stdout
