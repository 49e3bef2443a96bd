"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/k3oracle.c with one plausible error (a
swapped nibble, a dropped term, a wrong sign or index, a transposed operand),
built with gcc into a temporary directory. The pin suite is rerun against it
in a subprocess and must fail. Everything here runs on the CPU.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "k3oracle.c")

MUTANTS = {
    "nibble_order": ("return (k & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 15u);",
                     "return (k & 1) ? (uint32_t)(b & 15u) : (uint32_t)(b >> 4);"),
    "e2m1_mantissa": ("ldexp(1.0 + 0.5 * (double)m, (int)e - 1)",
                      "ldexp(1.0 + 0.25 * (double)m, (int)e - 1)"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * (double)m, (int)e - 1)",
                  "ldexp(1.0 + 0.5 * (double)m, (int)e)"),
    "e8m0_bias": ("return ldexp(1.0, (int)s - 127);", "return ldexp(1.0, (int)s - 128);"),
    "scale_block_16": ("acc += (k3o_e2m1(k3o_nibble(q, k)) * k3o_e8m0(s[k >> 5])) * x[k];",
                       "acc += (k3o_e2m1(k3o_nibble(q, k)) * k3o_e8m0(s[k >> 4])) * x[k];"),
    "bias_sign": ("l[e] += (double)bias[e];", "l[e] -= (double)bias[e];"),
    "router_transposed": ("const uint16_t* wr = w + (int64_t)k * E;\n      for (int32_t e = 0; e < E; ++e) l[e] += xk * bf16d(wr[e]);",
                          "for (int32_t e = 0; e < E; ++e) l[e] += xk * bf16d(w[(int64_t)e * d + k]);"),
    "softmax_no_max": ("p[e] = exp(l[e] - m);", "p[e] = exp(l[e]);"),
    "topk_tie_high_id": ("  return a < b;\n}", "  return a > b;\n}"),
    "gate_by_slot": ("gates[(int64_t)t * k + r] = p[ids[(int64_t)t * k + r]];",
                     "gates[(int64_t)t * k + r] = p[r];"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "swiglu_swapped": ("    h[j] = silu(u) * v;\n  }\n  const int64_t dq",
                       "    h[j] = u * silu(v);\n  }\n  const int64_t dq"),
    "combine_drops_gate": ("yt[i] += g * z[i];", "yt[i] += z[i] + 0.0 * g;"),
    "down_row_stride": ("const int64_t dq = f / 2, ds = f / 32;",
                        "const int64_t dq = f / 4, ds = f / 32;"),
    "rms_eps_outside": ("sqrt(ss / (double)d + eps)", "(sqrt(ss / (double)d) + eps)"),
    "bucket_unstable": ("for (int64_t p = 0; p < n; ++p) rows[next[ids[p]]++] = (int32_t)p;",
                        "for (int64_t p = n - 1; p >= 0; --p) rows[next[ids[p]]++] = (int32_t)p;"),
    "residual_dropped": ("yt[i] = (ht[i] + s[i]) + yt[i];", "yt[i] = s[i] + yt[i] + 0.0 * ht[i];"),
    "shared_down_transposed": ("a += bf16d(wd[(int64_t)i * f + j]) * h[j];",
                               "a += bf16d(wd[(int64_t)j * d + i]) * h[j];"),
}


def _run_mutant(name: str) -> tuple:
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    tmp = tempfile.mkdtemp(prefix=f"k3o_mut_{name}_")
    try:
        shutil.copy(os.path.join(ROOT, "oracle", "k3oracle.h"), tmp)
        with open(os.path.join(tmp, "k3oracle.c"), "w") as fh:
            fh.write(src.replace(old, new))
        r = subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
                            "-ffp-contract=off", "-o", "libmut.so", "k3oracle.c", "-lm"],
                           cwd=tmp, capture_output=True, text=True)
        if r.returncode != 0:
            return name, "build", r.stderr[-2000:]
        env = dict(os.environ, K3ORACLE_LIB=os.path.join(tmp, "libmut.so"), OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        return name, r.returncode, r.stdout[-600:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_every_planted_mistake_is_caught():
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_mutant, sorted(MUTANTS)))
    survivors = [(n, rc, out) for n, rc, out in results if rc == 0 or rc == "build"]
    assert not survivors, "mutants not caught:\n" + "\n".join(
        f"{n}: rc={rc}\n{out}" for n, rc, out in survivors)
