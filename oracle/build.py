"""Build the fp64 CPU oracle (test infrastructure) with gcc: plain C99, no
fast-math, no FMA contraction, OpenMP only across independent outputs."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
FLAGS = ["-O3", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-fno-fast-math",
         "-ffp-contract=off"]


def build(src: str = "k3oracle.c", out: str = "libk3oracle.so", cwd: str = HERE) -> str:
    cmd = ["gcc", *FLAGS, "-I", HERE, "-o", out, src, "-lm"]
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return os.path.join(cwd, out)


if __name__ == "__main__":
    build()
