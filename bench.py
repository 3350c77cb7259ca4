#!/usr/bin/env python3
"""Benchmark of the batched block-tridiagonal PCG / bdmv hot path on one GPU.

Prints ONE JSON line.  The headline (top-level ``value``) is batched PCG
solves/s on the streamed workload (fp32, state_size=21, knot_points=64, 2048
problems): one step = one ``glass_pcg_batched`` call that runs every step of
the path (strip loads, matvecs, dots, fused updates, stopping test, write-back)
for the whole batch.  The same run also times the other workloads (bdmv
ss=14/kp=64/8192 problems, PCG ss=6/kp=32/64 and ss=14/kp=32/4096, and the
grid-wide fp64 chain ss=12/kp=8192) and reports each under ``workloads`` with
its own roofline and CPU-oracle baseline.

Inputs are generated once, copied to HBM, and reused; each timed PCG step
starts from its own copy of x0 = 0 (prepared before the timed region), so no
step starts from an already-converged x.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor peak


def algorithmic_bytes_pcg(w, iters: np.ndarray, resident: bool) -> float:
    """Bytes one solve must move between HBM and the chip, by the algorithm:
    S and Pinv (n*3ss each) once if they stay on chip, else once per pass
    (the initial S x0 / Pinv r pass plus one per iteration); x read, b read,
    x written (n each); iters (4 bytes)."""
    es = np.dtype(w.dtype).itemsize
    mat = 2 * w.n * 3 * w.ss * es
    vec = 3 * w.n * es + 4
    passes = np.ones_like(iters, dtype=np.float64) if resident else (iters.astype(np.float64) + 1)
    return float(np.sum(passes * mat + vec))


def algorithmic_bytes_bdmv(w, B: int) -> float:
    es = np.dtype(w.dtype).itemsize
    return float(B) * (w.n * 3 * w.ss * es + (w.kp + 2) * w.ss * es + w.n * es)


def cpu_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def time_cpu(fn, budget_s: float):
    """Run fn() until ~budget_s has elapsed; return (seconds per call, calls)."""
    fn()  # warm
    t0 = time.perf_counter()
    calls = 0
    while True:
        fn()
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return el / calls, calls


class Timer:
    """HIP events on the stream the library launches on (torch's current
    stream): per-launch durations plus the whole timed region."""

    def __init__(self, torch, steps):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]

    def launch_ms(self):
        return [a.elapsed_time(b) for a, b in self.ev]


def bench_pcg(torch, glass, cfg, steps, warmup, cpu_budget, with_cpu):
    w = workloads.CONFIGS[cfg]
    inp = workloads.generate(w)
    dev = torch.device("cuda:0")
    S = torch.from_numpy(inp["S"]).to(dev)
    P = torch.from_numpy(inp["Pinv"]).to(dev)
    b = torch.from_numpy(inp["b"]).to(dev)
    B = w.n_problems
    xs = [torch.zeros((B, w.n), dtype=S.dtype, device=dev) for _ in range(steps + warmup)]
    iters = torch.zeros(B, dtype=torch.int32, device=dev)
    grid = cfg == 4
    if grid:
        ws = torch.empty(glass.pcg_grid_workspace_bytes(w.ss, w.kp, S.dtype),
                         dtype=torch.uint8, device=dev)

    def run(x):
        if grid:
            glass.pcg_grid(x, S, P, b, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, iters, ws)
        else:
            glass.pcg_batched(x, S, P, b, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, iters)

    for k in range(warmup):
        run(xs[steps + k])
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    t0 = time.perf_counter()
    for k in range(steps):
        tm.ev[k][0].record()
        run(xs[k])
        tm.ev[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = tm.launch_ms()
    it = iters.cpu().numpy()
    avg_ms = float(np.mean(launch_ms))
    resident = cfg in (0, 2, 4)
    nbytes = algorithmic_bytes_pcg(w, it, resident)
    out = {
        "workload": w.name, "kind": "grid_pcg" if grid else "batched_pcg",
        "dtype": np.dtype(w.dtype).name, "state_size": w.ss, "knot_points": w.kp,
        "n_problems": B, "solves_per_s": B * steps / wall, "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_avg": avg_ms, "kernel_ms_min": float(np.min(launch_ms)),
        "iterations": {str(k): int(v) for k, v in zip(*np.unique(it, return_counts=True))},
        "roofline": {"bound": "hbm", "achieved": nbytes / (avg_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes},
    }
    if grid:
        out["us_per_iteration"] = avg_ms * 1e3 / max(1, int(it[0]))
    if with_cpu:
        import oracle
        nt = 1 if grid else cpu_threads()
        prec = "f32" if w.dtype == np.float32 else "f64"
        sec, calls = time_cpu(lambda: oracle.pcg(inp["x0"], inp["S"], inp["Pinv"], inp["b"], w.ss,
                                                 w.kp, w.max_iters, w.rel_tol, w.abs_tol, prec, nt),
                              cpu_budget)
        out["cpu_baseline"] = {"value": B / sec, "unit": "solves/s", "cores": nt, "kind": "oracle",
                               "sample": "the full %d-problem workload, %d repetitions" % (B, calls)}
    return out


def bench_bdmv(torch, glass, steps, warmup, cpu_budget, with_cpu):
    w = workloads.CONFIGS[1]
    inp = workloads.generate(w)
    dev = torch.device("cuda:0")
    S = torch.from_numpy(inp["S"]).to(dev)
    v = torch.from_numpy(inp["v"]).to(dev)
    y = torch.zeros_like(v)
    for _ in range(warmup):
        glass.bdmv_batched(y, S, v, w.ss, w.kp)
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    t0 = time.perf_counter()
    for k in range(steps):
        tm.ev[k][0].record()
        glass.bdmv_batched(y, S, v, w.ss, w.kp)
        tm.ev[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = tm.launch_ms()
    avg_ms = float(np.mean(launch_ms))
    nbytes = algorithmic_bytes_bdmv(w, w.n_problems)
    out = {
        "workload": w.name, "kind": "bdmv", "dtype": "float32", "state_size": w.ss,
        "knot_points": w.kp, "n_problems": w.n_problems,
        "gb_per_s": nbytes / (wall / steps) / 1e9, "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_avg": avg_ms, "kernel_ms_min": float(np.min(launch_ms)),
        "roofline": {"bound": "hbm", "achieved": nbytes / (avg_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes},
    }
    if with_cpu:
        import oracle
        nt = cpu_threads()
        sample = 2048
        sec, calls = time_cpu(lambda: oracle.bdmv(inp["S"][:sample], inp["v"][:sample], w.ss, w.kp,
                                                  "f32", nthreads=nt), cpu_budget)
        out["cpu_baseline"] = {"value": algorithmic_bytes_bdmv(w, sample) / sec / 1e9,
                               "unit": "GB/s", "cores": nt, "kind": "oracle",
                               "sample": "%d of %d problems (float32 sums), %d repetitions"
                                         % (sample, w.n_problems, calls)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="all",
                    help="comma list of pcg0,bdmv1,pcg2,pcg3,grid4 or 'all' / 'primary'")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-budget", type=float, default=4.0,
                    help="seconds of oracle time per workload baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(problems are independent; see the sharding note in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_tridiagonal_pcg_bdmv_amd as glass
    glass.load()
    torch.cuda.set_device(0)

    names = {"pcg0": 0, "bdmv1": 1, "pcg2": 2, "pcg3": 3, "grid4": 4}
    if args.workloads == "all":
        sel = list(names)
    elif args.workloads == "primary":
        sel = ["pcg3"]
    else:
        sel = [s.strip() for s in args.workloads.split(",") if s.strip()]
    with_cpu = not args.no_cpu
    res = {}
    for name in sel:
        print("[bench] %s ..." % name, file=sys.stderr, flush=True)
        if names[name] == 1:
            res[name] = bench_bdmv(torch, glass, args.steps, args.warmup, args.cpu_budget, with_cpu)
        else:
            # the primary workload gets the larger CPU budget (10 s)
            budget = max(args.cpu_budget, 10.0) if name == "pcg3" else args.cpu_budget
            res[name] = bench_pcg(torch, glass, names[name], args.steps, args.warmup, budget,
                                  with_cpu)
        print("[bench] %s done: %s" % (name, json.dumps(res[name])[:300]), file=sys.stderr,
              flush=True)

    head = res.get("pcg3") or next(iter(res.values()))
    w = workloads.CONFIGS[3]
    line = {
        "metric": "PCG solves/sec (batched) and bdmv HBM GB/s as fraction of MI355X peak",
        "value": head.get("solves_per_s", head.get("gb_per_s")),
        "unit": "solves/s" if "solves_per_s" in head else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": head["workload"], "state_size": head["state_size"],
                   "knot_points": head["knot_points"], "n_problems": head["n_problems"],
                   "rel_tol": w.rel_tol, "max_iters": w.max_iters,
                   "parallelism": "one problem per workgroup"},
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "workloads": res,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
