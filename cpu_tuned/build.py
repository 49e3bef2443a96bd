"""Build the tuned CPU comparator with gcc: C99, OpenMP, no fast-math, no FMA contraction
(the AVX2 functions carry their own target attribute; the host check picks them)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
FLAGS = ["-O3", "-fPIC", "-shared", "-fopenmp", "-std=gnu99", "-fno-fast-math",
         "-ffp-contract=off"]


def build(src: str = "k3cpu.c", out: str = "libk3cpu.so", cwd: str = HERE) -> str:
    cmd = ["gcc", *FLAGS, "-I", HERE, "-o", out, src, "-lm"]
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"tuned CPU build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return os.path.join(cwd, out)


if __name__ == "__main__":
    build()
