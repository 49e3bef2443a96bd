"""Build the seeded input generator: host library (gcc) and device fill (hipcc)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(device: bool = True) -> None:
    _run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-ffp-contract=off",
          "-o", "libk3gen.so", "k3gen.c", "-lm"])
    if device:
        _run(["hipcc", *HIP_FLAGS, "-o", "libk3gen_dev.so", "k3gen_dev.hip"])


if __name__ == "__main__":
    build()
