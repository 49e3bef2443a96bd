#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

A step is one whole layer (router GEMV -> softmax/top-k -> bucket -> MXFP4 gate/up +
SwiGLU -> MXFP4 down + gate-weighted combine) over one batch of synthetic tokens,
through k3moe_layer_forward. Inputs sit in HBM before the timed region; each step
takes a fresh token set so routing (and the experts read) changes from step to step
and the 256 MB last-level cache cannot serve a repeated working set.

Prints ONE JSON line. `value` is the algorithmic weight stream of a step (the k
selected experts' MXFP4 bytes + the bf16 router) divided by the measured step time.
`roofline` reports the dominant kernel (the MXFP4 gate/up GEMV) timed live with HIP
events around its own launch; `cpu_baseline` times the fp64 CPU oracle on a small
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_MIN_TOKENS = 16  # the library's grouped-MFMA path starts at this many tokens
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


class Hip:
    """Minimal ctypes access to HIP events (on the stream the library launches on)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b) -> float:
        self.L.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def workload_desc(w) -> str:
    s = f"d={w.d} f={w.f} E={w.E} k={w.k} T={w.T}"
    if w.zipf_alpha:
        s += f" zipf={w.zipf_alpha}"
    return s


def expert_bytes_per_step(w, ids_np) -> int:
    """Algorithmic MXFP4 bytes: every distinct selected expert read once."""
    import numpy as np
    return int(len(np.unique(ids_np))) * w.expert_bytes


def capture_graph(fn):
    """One HIP graph of fn(), captured on a torch stream after an eager run of fn()."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_loop(args, step, nsets):
    """Warm-up, then exactly args.steps timed steps (eager, or graph replays with --graph);
    returns (t0, t1)."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        graphs = [capture_graph(lambda s=s: step(s)) for s in range(nsets)]
        for i in range(args.warmup):
            graphs[i % nsets].replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if args.graph:
            graphs[(args.warmup + i) % nsets].replay()
        else:
            step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t0, t1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def omp_threads() -> int:
    """Threads the OpenMP host code (oracle, tuned comparator) runs with."""
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(w, n_tokens: int, budget_s: float = 20.0):
    """Time the fp64 oracle on single-token layers of the same workload.

    Tokens run one at a time (their 16 experts drawn untimed before each), until
    `n_tokens` are done or `budget_s` seconds of oracle time are spent."""
    import numpy as np

    import oracle
    wr = w.router_w(0)
    bias = w.bias(0)
    sec, done = 0.0, 0
    for i in range(n_tokens):
        x = w.x_bf16(token_set=1000 + i, T=1)
        ids, _, _, _ = oracle.layer_route(x, wr, bias, w.k)
        experts = {int(e): w.expert_host(0, int(e)) for e in np.unique(ids)}
        t0 = time.perf_counter()
        oracle.layer_route(x, wr, bias, w.k)
        oracle.layer_forward(x, wr, bias, experts, w.d, w.f, w.E, w.k)
        sec += time.perf_counter() - t0
        done += 1
        if sec >= budget_s:
            break
    bytes_total = done * (w.k * w.expert_bytes + w.d * w.E * 2)
    return {"value": round(bytes_total / sec / 1e9, 4), "unit": "GB/s", "cores": omp_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} single-token decode layers ({workload_desc(w)}), fp64 oracle, "
                      f"{sec:.1f} s of oracle time"}


def cpu_baseline_prefill(w, n_tokens: int = 16, budget_s: float = 15.0):
    """The fp64 oracle on a bounded sample of the prefill chunk: `n_tokens` rows of the
    chunk's first token set, evenly spaced, each run as a one-token layer (router with the
    chunk's Zipf bias, its 16 experts drawn untimed before it). Useful SwiGLU flops
    (6 d f per routed pair) per second of oracle time."""
    import numpy as np

    import oracle
    wr = w.router_w(0)
    bias = w.bias(0)
    xall = w.x_bf16(token_set=0)
    rows = np.unique(np.linspace(0, w.T - 1, n_tokens).round().astype(int))
    sec, done = 0.0, 0
    for t in rows:
        x = np.ascontiguousarray(xall[t:t + 1])
        ids, _, _, _ = oracle.layer_route(x, wr, bias, w.k)
        experts = {int(e): w.expert_host(0, int(e)) for e in np.unique(ids)}
        t0 = time.perf_counter()
        oracle.layer_route(x, wr, bias, w.k)
        oracle.layer_forward(x, wr, bias, experts, w.d, w.f, w.E, w.k)
        sec += time.perf_counter() - t0
        done += 1
        if sec >= budget_s:
            break
    flops = done * 6.0 * w.d * w.f * w.k
    return {"value": round(flops / sec / 1e9, 3), "unit": "GFLOP/s", "cores": omp_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} of the {w.T} tokens of the prefill chunk ({workload_desc(w)}), "
                      f"evenly spaced, each as a one-token layer, fp64 oracle, {sec:.1f} s"}


def cpu_tuned_baseline(w, n_tokens: int, budget_s: float = 10.0):
    """Time the tuned CPU comparator (cpu_tuned/: AVX2 across outputs, OpenMP, equal to the
    oracle bit for bit) on single-token layers of the same workload, like cpu_baseline."""
    import numpy as np

    import cpu_tuned
    wr = w.router_w(0)
    bias = w.bias(0)
    sec, done = 0.0, 0
    for i in range(n_tokens):
        x = w.x_bf16(token_set=1000 + i, T=1)
        ids, _ = cpu_tuned.layer_route(x, wr, bias, w.k)  # untimed: which experts to draw
        experts = {int(e): w.expert_host(0, int(e)) for e in np.unique(ids)}
        t0 = time.perf_counter()
        cpu_tuned.layer_forward(x, wr, bias, experts, w.d, w.f, w.E, w.k)
        sec += time.perf_counter() - t0
        done += 1
        if sec >= budget_s:
            break
    bytes_total = done * (w.k * w.expert_bytes + w.d * w.E * 2)
    return {"value": round(bytes_total / sec / 1e9, 4), "unit": "GB/s", "cores": omp_threads(),
            "cpu": cpu_model(),
            "kind": "tuned CPU (AVX2 across outputs, OpenMP), equal to the oracle bit for bit"
                    if cpu_tuned.simd() else "tuned CPU (scalar host), equal to the oracle",
            "sample": f"{done} single-token decode layers ({workload_desc(w)}), "
                      f"{sec:.2f} s"}


DTYPE_DECODE = ("mxfp4 weights: gate/up bf16 x fp4->bf16 dot2 (fp32 acc), down block-scaled "
                "MFMA fp4 x 3 fp8(e4m3) terms of h (fp32 acc); router fp64")
DTYPE_GROUPED = ("mxfp4 weights on block-scaled MFMA: fp4 x 2 fp8(e4m3) terms of x (gate/up), "
                 "fp4 x 3 fp8(e4m3) terms of h (down), fp32 acc; router fp64")
DTYPE_GEMV = "mxfp4 weights: fp4->bf16/fp32 conversions, fp32 FMA/dot2 (fp32 acc); router fp64"


def dtype_of(w) -> str:
    if w.T == 1:
        return DTYPE_DECODE
    return DTYPE_GROUPED if w.T >= MFMA_MIN_TOKENS else DTYPE_GEMV


def use_packed(args, w) -> bool:
    """Expert layout of a layer leg: --layout if given (the default line's prefill leg
    follows it too), else the packed tile layout wherever the shape allows it (d % 1024 and
    f % 512; for one token also f <= 1536 and k <= 16, the one-token kernels' range)."""
    if args.layout:
        return args.layout == "packed"
    if w.d % 1024 or w.f % 512:
        return False
    return w.T > 1 or (w.f <= 1536 and w.k <= 16)


def spread(vals):
    import numpy as np
    v = np.asarray(vals, dtype=float)
    med = float(np.median(v))
    return {"ms_per_step": [round(float(a), 5) for a in v], "median": round(med, 5),
            "spread_pct": round(float((v.max() - v.min()) / med * 100.0), 2)}


_SWEEP = None


def clean_sweep():
    """Three read-only passes over a 2 GB buffer, enqueued right before the warm-up steps.

    Generating the resident inputs writes gigabytes, and the caches are left holding dirty
    lines; the first ~20 decode steps after such writes run 82-84 us instead of 72 us while
    those lines are written back (measured: the same steps right after a read-only sweep run
    at 72 us from the first one). The sweep leaves the caches clean and holding none of the
    layer's weights, the state a decode step meets after other decode steps."""
    import torch
    global _SWEEP
    if _SWEEP is None:
        _SWEEP = torch.ones(1 << 29, dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
    for _ in range(3):
        _SWEEP.sum()


class LayerLeg:
    """One bare MoE layer workload (decode, batched or prefill) resident on the GPU: its
    experts, router, bias, token sets, workspace and outputs, and one step =
    k3moe_layer_forward over the next token set."""

    def __init__(self, args, w, dev, packed=False):
        import torch

        import mxfp4_expert_matmul_k3moe_amd as k3
        from k3gen import device as gdev
        self.args, self.w, self.k3, self.packed = args, w, k3, packed
        self.dims = k3.make_dims(w.d, w.f, w.E, w.k)
        self.ex = k3.MxExperts(**gdev.experts(w, 0, dev))
        if packed:  # the packed tile layout, made once (weight preparation, not timed)
            rm = self.ex
            self.ex = k3.pack_experts(self.dims, rm)
            torch.cuda.synchronize()
            del rm
            torch.cuda.empty_cache()
        self.wr = gdev.router_w(w, 0, dev)
        self.bias = gdev.bias(w, 0, dev)
        # fresh tokens every step; prefill steps read most experts anyway, so fewer sets
        self.nsets = max(1, args.token_sets if w.T <= 64 else min(args.token_sets, 4))
        self.xs = torch.stack([gdev.x_bf16(w, token_set=i, device=dev)
                               for i in range(self.nsets)])
        self.ws = k3.make_workspace(self.dims, w.T, dev)
        self.y = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)
        self.ybf = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
        self.ids = torch.empty((self.nsets, w.T, w.k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)

    def step(self, i):
        s = i % self.nsets
        fwd = self.k3.layer_forward_packed if self.packed else self.k3.layer_forward
        fwd(self.dims, self.xs[s], self.wr, self.bias, self.ex, y=self.y, y_bf16=self.ybf,
            ids=self.ids[s], gates=self.gates, ws=self.ws)

    def measure(self, repeats: int) -> dict:
        """A read-only sweep (see clean_sweep), W warm-up steps, exactly K timed steps, then
        `repeats` more timed runs of K steps (for median and spread), then the dominant
        kernels timed live by HIP events."""
        import numpy as np
        import torch
        args, w, k3 = self.args, self.w, self.k3
        clean_sweep()
        t0, t1 = timed_loop(args, self.step, self.nsets)
        runs = [(t1 - t0) * 1e3 / args.steps]
        for r in range(repeats):
            torch.cuda.synchronize()
            a = time.perf_counter()
            for i in range(args.steps):
                self.step(args.warmup + i)
            torch.cuda.synchronize()
            runs.append((time.perf_counter() - a) * 1e3 / args.steps)
        ids_np = self.ids.cpu().numpy()
        uniq = [len(np.unique(ids_np[s2])) for s2 in range(self.nsets)]
        step_sets = [(args.warmup + i) % self.nsets for i in range(args.steps)]
        hip = Hip()
        nprobe = min(args.steps, 100 if w.T <= 64 else 20)
        kern = {}
        for which, name in ((k3.KERNEL_GATE_UP, "gate_up"), (k3.KERNEL_DOWN, "down")):
            evs = [(hip.event(), hip.event()) for _ in range(nprobe)]
            for i in range(nprobe):
                k3.time_next_kernel(which, evs[i][0], evs[i][1])
                self.step(args.warmup + i)
            torch.cuda.synchronize()
            times = [hip.elapsed_ms(a, b) for a, b in evs]
            for a, b in evs:
                hip.destroy(a)
                hip.destroy(b)
            kern[name] = sum(times) / len(times)
        sel = float(np.mean([uniq[(args.warmup + i) % self.nsets] for i in range(nprobe)]))
        return {"sec": t1 - t0, "ms_per_step": runs[0], "runs": runs, "uniq": uniq,
                "bytes_timed": sum(uniq[s2] * w.expert_bytes + w.d * w.E * 2
                                   for s2 in step_sets),
                "gate_up_ms": kern["gate_up"], "down_ms": kern["down"], "sel": sel}


def grouped_label(packed: bool) -> str:
    return ("mfma_ffn_kernel<gate/up> (grouped GEMM, block-scaled FP4 x FP8 MFMA, two FP8 "
            "token terms, + SwiGLU; " + ("packed tile layout, 1 KB per weight tile step)"
                                        if packed else "row-major weights)"))


def decode_like_fields(w, m, traffic, packed=False):
    """value / roofline / kernels of a weight-stream (T <= 64) workload."""
    import numpy as np
    value = m["bytes_timed"] / m["sec"] / 1e9
    gu_bytes = m["sel"] * 2 * w.f * (w.d // 2 + w.d // 32)
    dn_bytes = m["sel"] * w.d * (w.f // 2 + w.f // 32)
    ach = gu_bytes / (m["gate_up_ms"] * 1e-3) / 1e9
    if w.T == 1:
        kname = ("gateup_decode_packed_kernel (MXFP4 gate/up + SwiGLU, one token, packed tile "
                 "layout, block-scaled FP4 x FP8 MFMA on the token's E4M3 terms)"
                 if packed else "gateup_decode_kernel (MXFP4 gate/up GEMV + SwiGLU)")
    elif w.T >= MFMA_MIN_TOKENS or packed:
        kname = grouped_label(packed)
    else:
        kname = "gateup_gemv_kernel (MXFP4 gate/up GEMV + SwiGLU)"
    roof = {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": int(gu_bytes), "avg_launch_us": round(m["gate_up_ms"] * 1e3, 2)}
    extra = {"down_us": round(m["down_ms"] * 1e3, 2),
             "down_GBps": round(dn_bytes / (m["down_ms"] * 1e-3) / 1e9, 1),
             "experts_GBps": round((gu_bytes + dn_bytes) /
                                   ((m["gate_up_ms"] + m["down_ms"]) * 1e-3) / 1e9, 1),
             "layer_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
             "distinct_experts_per_step": round(float(np.mean(m["uniq"])), 1)}
    return value, "GB/s", roof, extra


def prefill_fields(w, m, traffic, packed=False):
    """value / roofline / kernels of a grouped-GEMM (prefill) workload."""
    import numpy as np
    pairs = w.T * w.k
    value = 6.0 * w.d * w.f * pairs / (m["ms_per_step"] * 1e-3) / 1e12
    gu_flops = 4.0 * w.d * w.f * pairs
    dn_flops = 2.0 * w.d * w.f * pairs
    gu_s, dn_s = m["gate_up_ms"] * 1e-3, m["down_ms"] * 1e-3
    gu_bytes = m["sel"] * 2 * w.f * (w.d // 2 + w.d // 32)
    dn_bytes = m["sel"] * w.d * (w.f // 2 + w.f // 32)
    ach = gu_flops / gu_s / 1e12
    floor_ms = float(np.mean(m["uniq"])) * w.expert_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    # two FP8-rate MFMAs (5.0 PFLOP/s) per useful product: 2.5 PFLOP/s of useful flops,
    # the same ceiling as bf16 MFMA
    roof = {"bound": "mfma",
            "kernel": grouped_label(packed),
            "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "flops_per_launch": gu_flops, "avg_launch_us": round(m["gate_up_ms"] * 1e3, 2),
            "weight_bytes_per_launch": int(gu_bytes),
            "hbm_GBps": round(gu_bytes / gu_s / 1e9, 1),
            "hbm_frac": round(gu_bytes / gu_s / 1e9 / HBM_PEAK_GBS, 4)}
    extra = {"down_us": round(m["down_ms"] * 1e3, 2),
             "down_TFLOPs": round(dn_flops / dn_s / 1e12, 1),
             "down_frac_of_mfma_peak": round(dn_flops / dn_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
             "down_hbm_GBps": round(dn_bytes / dn_s / 1e9, 1),
             "layer_frac_of_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
             "weight_GBps": round(m["bytes_timed"] / m["sec"] / 1e9, 1),
             "distinct_experts_per_step": round(float(np.mean(m["uniq"])), 1),
             "hbm_floor_ms": round(floor_ms, 3),
             "frac_of_hbm_floor": round(floor_ms / m["ms_per_step"], 4)}
    return value, "TFLOP/s", roof, extra


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "batched", "batched_zipf", "prefill", "stack8",
                             "cached"])
    ap.add_argument("--slots", type=int, default=128,
                    help="cached workload: HBM expert slots (the other experts stay in "
                         "pinned host memory)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count (e.g. a prefill chunk sweep)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 20 times (counter scale)")
    ap.add_argument("--token-sets", type=int, default=64)
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--repeats", type=int, default=3,
                    help="extra timed runs of --steps steps after the first, for the median "
                         "and spread")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode: leave out the prefill leg of the default line")
    ap.add_argument("--hot-tokens", type=int, default=None,
                    help="k3moe_set_hot_tokens before the run: experts with fewer tokens in a "
                         "step read their weights non-temporally in the grouped kernels "
                         "(0..16; the library's default is 16)")
    ap.add_argument("--layout", choices=["rowmajor", "packed"], default=None,
                    help="expert weight layout of a single-workload run (default: packed "
                         "wherever the shape allows it)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one HIP graph per token set (captured on the "
                         "caller's stream) instead of eager calls")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library runs the layer on a single GPU "
              "(expert-parallel sharding across GPUs is not implemented); use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * 1000 * 1000
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 20}), flush=True)
        return 0

    from k3gen.workloads import WORKLOADS

    w = WORKLOADS["decode" if args.workload == "cached" else args.workload]
    if args.hot_tokens is not None:
        import mxfp4_expert_matmul_k3moe_amd as k3
        k3.set_hot_tokens(args.hot_tokens)
    if args.tokens:
        w = w.with_(T=args.tokens)
    if args.workload == "cached":
        return bench_cached(args, w)
    if w.block:
        return bench_stack(args, w)
    dev = torch.device("cuda:0")
    metric = "MoE layer MXFP4 weight-stream GB/s (decode) + TFLOP/s (prefill), % of peak"
    # the default line carries both halves of the metric: the prefill chunk (config 4) runs
    # first, then the decode headline; CPU baselines run before any GPU work
    with_prefill = (args.workload == "decode" and not args.tokens and not args.no_prefill
                    and not args.graph)
    cpu = {}
    if not args.no_cpu_baseline:
        if w.T == 1:
            cpu["base"] = cpu_baseline(w, args.cpu_tokens)
            cpu["tuned"] = cpu_tuned_baseline(w, args.cpu_tokens)
        if with_prefill or (w.T > 64 and not args.tokens):
            cpu["prefill"] = cpu_baseline_prefill(WORKLOADS["prefill"])

    prefill_obj = None
    if with_prefill:
        wp = WORKLOADS["prefill"]
        leg = LayerLeg(args, wp, dev, packed=use_packed(args, wp))
        mp = leg.measure(args.repeats)
        del leg
        torch.cuda.empty_cache()
        pk = use_packed(args, wp)
        v, unit, roof, extra = prefill_fields(wp, mp, grouped_traffic(wp, pk), pk)
        prefill_obj = {"value": round(v, 2), "unit": unit, "steps": args.steps,
                       "warmup": args.warmup, "ms_per_step": round(mp["ms_per_step"], 5),
                       "repeats": spread(mp["runs"]), "dtype": dtype_of(wp),
                       "config": {"workload": f"{wp.name}: {workload_desc(wp)}",
                                  "token_sets": min(args.token_sets, 4),
                                  "expert_layout": "packed" if use_packed(args, wp)
                                  else "row-major"},
                       "roofline": roof, "kernels": extra,
                       "cpu_baseline": cpu.get("prefill")}

    leg = LayerLeg(args, w, dev, packed=use_packed(args, w))
    m = leg.measure(args.repeats)
    if w.T <= 64:
        traffic = (decode_traffic(leg.packed) if args.workload == "decode" and not args.tokens
                   else None)
        value, unit, roof, extra = decode_like_fields(w, m, traffic, leg.packed)
    else:
        value, unit, roof, extra = prefill_fields(w, m, grouped_traffic(w, leg.packed),
                                                  leg.packed)

    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(w),
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {workload_desc(w)}",
                   "bytes_per_step": int(round(m["bytes_timed"] / args.steps)),
                   "token_sets": leg.nsets, "hip_graph": bool(args.graph),
                   "expert_layout": "packed" if leg.packed else "row-major",
                   "hot_tokens": _hot_tokens(),
                   "preceded_by": ("the prefill leg below, then " if prefill_obj else "") +
                   "a 6 GB read-only sweep (no dirty lines from input generation in the "
                   "caches; none of the layer's weights in them)"},
        "repeats": spread(m["runs"]),
        "roofline": roof,
        "kernels": extra,
        "cpu_baseline": cpu.get("base") if w.T == 1 else cpu.get("prefill"),
    }
    if "tuned" in cpu:
        out["cpu_tuned"] = cpu["tuned"]
    if prefill_obj is not None:
        out["prefill"] = prefill_obj
    print(json.dumps(out), flush=True)
    return 0


def _hot_tokens() -> int:
    import mxfp4_expert_matmul_k3moe_amd as k3
    return k3.hot_tokens()


def _read_record(name: str) -> dict:
    path = os.path.join(ROOT, "profiles", name)
    tr = {}
    if os.path.exists(path):
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    tr[key.strip()] = val.strip()
    return tr


def decode_traffic(packed=False):
    """HBM bytes per launch of the T=1 gate/up kernel of that layout from the committed
    FETCH_SIZE / WRITE_SIZE record, used only while the kernel source it was measured on is
    unchanged."""
    tr = _read_record("gateup_decode_packed_traffic.txt" if packed
                      else "gateup_decode_traffic.txt")
    if not tr or tr.get("kernel_source_hash") != _kernel_hash(packed):
        return None
    return int(tr["bytes_per_launch"])


def grouped_traffic(w, packed):
    """HBM bytes per launch of the grouped gate/up GEMM on the prefill chunk (T=2048, Zipf
    bias) from the committed counter record of that layout, while the grouped-GEMM source is
    unchanged."""
    if w.name != "prefill" or w.T != 2048:
        return None
    tr = _read_record("gateup_grouped_packed_traffic.txt" if packed
                      else "gateup_grouped_traffic.txt")
    if not tr or tr.get("kernel_source_hash") != _grouped_hash():
        return None
    return int(tr["bytes_per_launch"])


def _grouped_hash() -> str:
    """Hash of the grouped-GEMM source (ffn_mfma.hip and k3moe_device.h)."""
    import hashlib
    csrc = os.path.join(ROOT, "mxfp4_expert_matmul_k3moe_amd", "csrc")
    h = hashlib.sha256()
    for n in ("ffn_mfma.hip", "k3moe_device.h"):
        with open(os.path.join(csrc, n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def bench_stack(args, w) -> int:
    """Config 5: one token through `w.layers` resident blocks (RMSNorm -> routed MoE + bf16
    shared SwiGLU -> residual), the fp32 residual chained from block to block. `value` =
    per-token weight stream (per block: k selected experts + router + shared expert) / step
    time."""
    import numpy as np
    import torch

    import mxfp4_expert_matmul_k3moe_amd as k3
    from k3gen import device as gdev

    dev = torch.device("cuda:0")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    # packed by default: the fp32-token gate/up of the packed layout holds 128 registers,
    # the row-major one 177
    packed = args.layout == "packed" or (args.layout is None and w.d % 1024 == 0 and
                                          w.f % 512 == 0)
    fwd = k3.layer_forward_packed if packed else k3.layer_forward
    layers = []
    for l in range(w.layers):
        ex = k3.MxExperts(**gdev.experts(w, l, dev))
        if packed:  # the packed copy, made once per layer (weight preparation, not timed)
            rm = ex
            ex = k3.pack_experts(dims, rm)
            torch.cuda.synchronize()
            del rm
            torch.cuda.empty_cache()
        b = gdev.block_extras(w, l, dev)
        blk = k3.BlockWeights(b["rms_gamma"], b["sh_gate"], b["sh_up"], b["sh_down"], 1e-6)
        layers.append((gdev.router_w(w, l, dev), gdev.bias(w, l, dev), ex, blk))
    nsets = max(1, min(args.token_sets, 16))
    h0 = torch.stack([torch.from_numpy(w.resid0(token_set=i)).to(dev) for i in range(nsets)])
    ws = k3.make_workspace(dims, w.T, dev)
    hb = [torch.empty((w.T, w.d), dtype=torch.float32, device=dev) for _ in range(2)]
    ids = torch.empty((w.layers, w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)

    def step(i):
        h = h0[i % nsets]
        for l, (wr, bias, ex, blk) in enumerate(layers):
            y = hb[l % 2]
            fwd(dims, h, wr, bias, ex, blk, y=y, ids=ids[l], gates=gates, ws=ws)
            h = y

    clean_sweep()
    t0, t1 = timed_loop(args, step, nsets)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ids_np = ids.cpu().numpy()
    distinct = [len(np.unique(ids_np[l])) for l in range(w.layers)]
    router_bytes, shared_bytes = w.d * w.E * 2, 3 * w.d * w.f * 2
    bytes_step = sum(n * w.expert_bytes + router_bytes + shared_bytes for n in distinct)

    hip = Hip()
    nprobe = min(args.steps, 50)
    kern = {}
    for which, name in ((k3.KERNEL_GATE_UP, "gate_up"), (k3.KERNEL_DOWN, "down")):
        evs = [(hip.event(), hip.event()) for _ in range(nprobe)]
        for i in range(nprobe):
            k3.time_next_kernel(which, evs[i][0], evs[i][1])  # the first block's launch
            step(args.warmup + i)
        torch.cuda.synchronize()
        times = [hip.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            hip.destroy(a)
            hip.destroy(b)
        kern[name] = sum(times) / len(times)
    gu_bytes = w.k * 2 * w.f * (w.d // 2 + w.d // 32)
    dn_bytes = w.k * w.d * (w.f // 2 + w.f // 32)
    # packed experts at these shapes: the gate/up launch also runs the shared expert's bf16
    # down GEMV (its d x f weights are part of that launch's bytes)
    shared_in_gu = packed and 256 < w.E <= 4096 and w.E % 8 == 0 and w.d <= 8192
    if shared_in_gu:
        gu_bytes += w.d * w.f * 2
    value = bytes_step * args.steps / (t1 - t0) / 1e9
    ach = gu_bytes / (kern["gate_up"] * 1e-3) / 1e9
    out = {
        "metric": "MoE layer MXFP4 weight-stream GB/s (decode) + TFLOP/s (prefill), % of peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_DECODE.replace("gate/up bf16", "gate/up fp32 x") +
                 "; shared expert bf16 weights x fp32 (fp32 acc)",
        "data": "synthetic",
        "config": {"workload": f"stack8: {workload_desc(w)} layers={w.layers}, block "
                               "(RMSNorm, shared expert, residual)",
                   "bytes_per_step": int(bytes_step), "token_sets": nsets,
                   "hip_graph": bool(args.graph),
                   "expert_layout": "packed" if packed else "row-major"},
        "roofline": {"bound": "hbm",
                     "kernel": ("gateup_packed_shared_down_kernel<fp32 x> (MXFP4 gate/up + "
                                "SwiGLU on the block-scaled MFMA, packed tile layout, and the "
                                "shared expert's bf16 down GEMV in the same launch)"
                                if shared_in_gu else
                                "gateup_decode_packed_kernel<fp32 x> (MXFP4 gate/up + "
                                "SwiGLU, packed tile layout)" if packed else
                                "gateup_decode_kernel<fp32 x> (MXFP4 gate/up GEMV + SwiGLU)"),
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     # the counter record was taken on the bf16-token instantiation
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(gu_bytes),
                     "avg_launch_us": round(kern["gate_up"] * 1e3, 2)},
        "kernels": {"down_us": round(kern["down"] * 1e3, 2),
                    "down_GBps": round(dn_bytes / (kern["down"] * 1e-3) / 1e9, 1),
                    "layer_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                    "us_per_block": round(ms_per_step * 1e3 / w.layers, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_cached(args, w) -> int:
    """Routed experts beyond HBM: the decode layer with all E experts in pinned host memory
    and `--slots` of them in HBM (k3moe_layer_forward_cached: router, routed ids to the
    host, LRU slot plan, host -> HBM copies of the misses, experts from the slots). A step
    is one fresh token set; its time includes the host round trip and the copies. `value` =
    the step's algorithmic weight stream (distinct selected experts + router) / step time,
    i.e. the PCIe-inclusive rate; the plain pinned host -> device copy rate measured in the
    same run is the ceiling of the copies."""
    import numpy as np
    import torch

    import mxfp4_expert_matmul_k3moe_amd as k3
    from k3gen import device as gdev

    dev = torch.device("cuda:0")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    C = max(w.k, min(args.slots, w.E))
    ex_dev = gdev.experts(w, 0, dev)
    host = {}
    for n in list(ex_dev):
        t = ex_dev.pop(n)
        h = torch.empty(t.shape, dtype=torch.uint8, pin_memory=True)
        h.copy_(t)
        host[n] = h
        del t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    host_ex = k3.MxExperts(**host)
    slots = k3.MxExperts(**{n: torch.empty((C,) + tuple(t.shape[1:]), dtype=torch.uint8,
                                           device=dev) for n, t in host.items()})
    cache = k3.ExpertCache(w.E, C, w.T * w.k)
    wr = gdev.router_w(w, 0, dev)
    bias = gdev.bias(w, 0, dev)
    nsets = max(1, args.token_sets)
    xs = torch.stack([gdev.x_bf16(w, token_set=i, device=dev) for i in range(nsets)])
    ws = k3.make_workspace(dims, w.T, dev)
    y = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)
    ids = torch.empty((nsets, w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    stats = []

    def step(i):
        s2 = i % nsets
        _, st = k3.layer_forward_cached(dims, xs[s2], wr, bias, host_ex, slots, cache, y=y,
                                        ids=ids[s2], gates=gates, ws=ws)
        stats.append((st.hits, st.misses, st.bytes_copied, st.distinct))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stats.clear()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = t1 - t0
    hits = sum(a[0] for a in stats)
    misses = sum(a[1] for a in stats)
    copied = sum(a[2] for a in stats)
    distinct = sum(a[3] for a in stats)
    bytes_timed = distinct * w.expert_bytes + args.steps * w.d * w.E * 2

    # the link itself: 1 GB pinned host -> device, 5 copies
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    link = 5 * n / (time.perf_counter() - c0) / 1e9
    h2d = copied / sec / 1e9
    out = {
        "metric": "MoE layer MXFP4 weight-stream GB/s (decode) + TFLOP/s (prefill), % of peak",
        "value": round(bytes_timed / sec / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_DECODE,
        "data": "synthetic",
        "config": {"workload": f"cached decode: {workload_desc(w)}, {w.E} experts in pinned "
                               f"host memory, {C} HBM slots, LRU",
                   "slots": C, "token_sets": nsets},
        "roofline": {"bound": "host link", "achieved": round(h2d, 2),
                     "peak": round(link, 2), "unit": "GB/s",
                     "frac": round(h2d / link, 4) if link > 0 else None, "traffic": None,
                     "note": "expert bytes copied host -> HBM per second of step time; peak = "
                             "plain 1 GB pinned host -> device copy in the same run"},
        "kernels": {"hit_rate": round(hits / max(hits + misses, 1), 4),
                    "misses_per_step": round(misses / args.steps, 2),
                    "distinct_experts_per_step": round(distinct / args.steps, 2),
                    "copied_MB_per_step": round(copied / args.steps / 1e6, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    # hand the pinned host memory (all E experts, ~15.7 GB at K3 size) back to the HIP
    # runtime before the interpreter exits, rather than from torch's allocator finalisers
    torch.cuda.synchronize()
    del host_ex, src
    host.clear()
    torch._C._host_emptyCache()
    return 0


def _function_text(src: str, marker: str) -> str:
    """Source of the top-level function whose signature contains `marker`: from the
    template line above it (if any) to its closing brace at column 0."""
    i = src.index(marker)
    start = src.rfind("\n", 0, i) + 1
    prev = src.rfind("\n", 0, start - 1) + 1
    if src[prev:start].startswith("template"):
        start = prev
    end = src.index("\n}\n", i) + 3
    return src[start:end]


def _kernel_hash(packed=False) -> str:
    """Hash of the T=1 gate/up kernel's own source (row-major or packed layout): its template,
    its launcher and the device helpers it uses (the traffic record holds while these are
    unchanged)."""
    import hashlib
    csrc = os.path.join(ROOT, "mxfp4_expert_matmul_k3moe_amd", "csrc")
    with open(os.path.join(csrc, "ffn_mfma.hip" if packed else "ffn_gemv.hip")) as fh:
        src = fh.read()
    h = hashlib.sha256()
    if packed:
        h.update(_function_text(src, "void gateup_decode_packed_kernel(").encode())
        h.update(_function_text(src, "hipError_t launch_gateup_decode_packed(").encode())
    else:
        h.update(_function_text(src, "void gateup_decode_kernel(").encode())
        h.update(_function_text(src, "hipError_t launch_gateup_decode(").encode())
    with open(os.path.join(csrc, "k3moe_device.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
