#!/usr/bin/env python3
"""Benchmark of the batched block-tridiagonal PCG / bdmv hot path on one GPU.

Prints ONE JSON line.  The headline (top-level ``value``) is batched PCG
solves/s on the streamed workload (fp32, state_size=21, knot_points=64, 2048
problems): one step = one ``glass_pcg_batched`` call that runs every step of
the path (strip loads, matvecs, dots, fused updates, stopping test, write-back)
for the whole batch.  The same run also times the other workloads (bdmv
ss=14/kp=64/8192 problems, PCG ss=6/kp=32/64 and ss=14/kp=32/4096, and the
grid-wide fp64 chain ss=12/kp=8192) and reports each under ``workloads`` with
its own roofline and CPU-oracle baseline, as does the direct solve
(``glass_bdsv_batched``) of the ss=14/kp=32/4096 systems.

Inputs are generated once, copied to HBM, and reused; each timed PCG step
starts from its own copy of x0 = 0 (prepared before the timed region), so no
step starts from an already-converged x.

Roofline: ``achieved`` = algorithmic bytes per launch / mean launch duration
(HIP events before the first and after the last timed launch, on the stream
the library launches on, divided by the number of launches).
``traffic`` = HBM bytes per launch of the workload's kernel measured by the
rocprofv3 FETCH_SIZE / WRITE_SIZE counters and calibrated against a copy of
known size; it is read from ``profiles/hbm_traffic.md`` and reported only
while the kernel sources still hash to the value recorded there (else null).

Other modes:
  --calibration-copy     also run a 1 GiB negation (read 1 GiB, write 1 GiB)
                         whose counters calibrate FETCH_SIZE / WRITE_SIZE
  --summarize-pmc F W    turn the two counter CSVs of rocprofv3 runs (F:
                         FETCH_SIZE, W: WRITE_SIZE) into profiles/hbm_traffic.md
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
CALIBRATION_BYTES = 1 << 30
METRIC = "PCG solves/sec (batched) and bdmv HBM GB/s as fraction of MI355X peak"

# The kernel each workload spends its time in (a substring of the demangled
# name rocprofv3 reports).
KERNEL_OF = {
    "pcg0": "pcg_batched_kernel<float, 6, 1, 10>",
    "bdmv1": "bdmv_kernel<float, 14>",
    "pcg2": "pcg_batched_kernel<float, 14, 1, 10>",
    "pcg3": "pcg_batched_kernel<float, 21, 3, 7>",
    "pcg3_stream": "pcg_batched_kernel<float, 21, 3, 1>",
    "grid4": "pcg_grid_kernel<double, 12,",
    "bdsv2": "bdsv_rows_kernel<float, 14,",
    "pcg2_f64": "pcg_batched_kernel<double, 14, 1, 7>",
    "grid4_f32": "pcg_grid_kernel<float, 12,",
    "pcg2_pd": "pcg_batched_kernel<float, 14, 2, 3>",
    "pcg3_pd": "pcg_batched_kernel<float, 21, 3, 9>",
    "pcg2_pdp": "pcg_batched_kernel<float, 14, 2, 6>",
    "pcg3_pdp": "pcg_batched_kernel<float, 21, 3, 8>",
    "grid4_sr": "pcg_grid_cg1_kernel<double, 12,",
    "grid4_f32_sr": "pcg_grid_cg1_kernel<float, 12,",
    "pcg0_multi": "pcg_multi_kernel<float, 6, 32, 6>",
    "pcg0_b4096": "pcg_batched_kernel<float, 6, 1, 10>",
    "pcg0_b4096_multi": "pcg_multi_kernel<float, 6, 32, 6>",
    "pcg3_unaligned": "pcg_batched_kernel<float, 21, 3, 7>",
}
# Workload inputs: the five configurations; bdsv2 is the direct solve of the
# same systems as pcg2 (ss=14, kp=32, 4096 problems); pcg2_f64 and grid4_f32
# are the precision variants of pcg2 and grid4 (same recipe and seeds).
CONFIG_OF = {"pcg0": 0, "bdmv1": 1, "pcg2": 2, "pcg3": 3, "pcg3_stream": 3, "grid4": 4, "bdsv2": 2,
             "pcg2_f64": 2, "grid4_f32": 4, "pcg2_pd": 2, "pcg3_pd": 3, "pcg2_pdp": 2,
             "pcg3_pdp": 3, "grid4_sr": 4, "grid4_f32_sr": 4, "pcg0_multi": 0, "pcg0_b4096": 0,
             "pcg0_b4096_multi": 0, "pcg3_unaligned": 3}
# Workloads run with GLASS_PCG_PINV_BLOCK_DIAGONAL (their Pinv is block-Jacobi,
# so the assertion holds): pcg2_pd and pcg3_pd are the ss=14 and ss=21
# workloads with the hint.
PINV_DIAG = {"pcg2_pd", "pcg3_pd"}
# Workloads run with GLASS_PCG_PINV_DIAGONAL_BLOCKS: the same systems with
# Pinv passed as its packed D blocks [B, kp, ss, ss].
PINV_PACKED = {"pcg2_pdp", "pcg3_pdp"}
# Workloads run with the S-resident placement switched off
# (GLASS_AMD_PCG_NO_HYBRID=1): pcg3_stream is the ss=21 workload with S and
# Pinv both streamed, the placement the S-resident one replaced.
NO_HYBRID = {"pcg3_stream"}
# Workloads run with several problems per wave (GLASS_AMD_PCG_MULTI=1): the
# ss=6 systems at their 64 problems and at 4096 (pcg0_b4096 is the same 4096
# problems in the default workgroup placement).
MULTI = {"pcg0_multi", "pcg0_b4096_multi"}
# Workloads whose matrices sit at addresses aligned to the element size only
# (4 bytes past a 16-byte boundary): the S-resident placement loads such rows
# from the 16-byte boundary below them, so this row checks that it costs
# nothing against the aligned pcg3.
UNALIGNED = {"pcg3_unaligned"}
# Grid workloads run in the single-reduction form (GLASS_GRID_SINGLE_REDUCTION).
SINGLE_RED = {"grid4_sr", "grid4_f32_sr"}
VARIANT_OF = {
    "grid4_sr": dict(name="grid_pcg_ss12_kp8192_f64_single_reduction"),
    "grid4_f32_sr": dict(name="grid_pcg_ss12_kp8192_f32_single_reduction", dtype=np.float32,
                         rel_tol=1e-7),
    "pcg2_pd": dict(name="pcg_ss14_kp32_b4096_f32_pinv_blockdiag"),
    "pcg3_pd": dict(name="pcg_ss21_kp64_b2048_f32_pinv_blockdiag"),
    "pcg3_stream": dict(name="pcg_ss21_kp64_b2048_f32_streamed"),
    "pcg2_pdp": dict(name="pcg_ss14_kp32_b4096_f32_pinv_diagonal_blocks"),
    "pcg3_pdp": dict(name="pcg_ss21_kp64_b2048_f32_pinv_diagonal_blocks"),
    "pcg2_f64": dict(name="pcg_ss14_kp32_b4096_f64", dtype=np.float64),
    "pcg0_multi": dict(name="pcg_ss6_kp32_b64_f32_several_per_wave"),
    "pcg0_b4096": dict(name="pcg_ss6_kp32_b4096_f32", n_problems=4096),
    "pcg0_b4096_multi": dict(name="pcg_ss6_kp32_b4096_f32_several_per_wave", n_problems=4096),
    "pcg3_unaligned": dict(name="pcg_ss21_kp64_b2048_f32_element_aligned"),
    "grid4_f32": dict(name="grid_pcg_ss12_kp8192_f32", dtype=np.float32, rel_tol=1e-7),
}


def workload_of(key):
    from dataclasses import replace
    w = workloads.WORKLOADS[CONFIG_OF[key]]
    return replace(w, **VARIANT_OF[key]) if key in VARIANT_OF else w


def code_without_comments(text: str) -> str:
    """C/C++ source with // and /* */ comments removed (string and character
    literals kept as they are) and blank lines and trailing blanks dropped,
    so that edits of comments alone, however many lines they take, do not
    change the hash below."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).splitlines() if line.strip())


def kernel_source_hash() -> str:
    """sha256 over the code of the HIP sources and the C ABI header (sorted by
    name, comments removed)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_tridiagonal_pcg_bdmv_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".hip", ".hpp")))
    files.append(os.path.join(ROOT, "include", "glass_amd.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(code_without_comments(fh.read()).encode())
    return h.hexdigest()


def algorithmic_bytes_pcg(w, iters: np.ndarray, resident, pinv_diag=False,
                          pass_rows=None) -> float:
    """Bytes one solve must move between HBM and the chip, by the algorithm:
    S and Pinv (n*3ss each; Pinv n*ss when only its D blocks are read) once
    if they stay on chip, else once per pass (the initial S x0 / Pinv r pass
    plus one per iteration); x read, b read, x written (n each); iters
    (4 bytes).  resident: True (both on chip), False (both streamed) or "S"
    (S on chip once; Pinv rows as the placement reads them: pass_rows =
    (rows at pass 0, at odd passes, at even passes >= 2), default every row
    at every pass)."""
    es = np.dtype(w.dtype).itemsize
    s_bytes = w.n * 3 * w.ss * es
    row_b = (w.ss if pinv_diag else 3 * w.ss) * es
    p_bytes = w.n * row_b
    vec = 3 * w.n * es + 4
    it = iters.astype(np.int64)
    passes = it.astype(np.float64) + 1
    if resident == "S":
        r0, r_odd, r_even = pass_rows if pass_rows is not None else (w.n, w.n, w.n)
        rows = r0 + ((it + 1) // 2) * r_odd + (it // 2) * r_even
        return float(np.sum(s_bytes + rows.astype(np.float64) * row_b + vec))
    if resident:
        passes = np.ones_like(passes)
    return float(np.sum(passes * (s_bytes + p_bytes) + vec))


def compulsory_bytes_pcg(w, B: int, pinv_diag=False) -> float:
    """Bytes every placement must move per launch: S and Pinv once (Pinv's D
    blocks only when only they are read), x read, b read, x written, iters."""
    es = np.dtype(w.dtype).itemsize
    s_bytes = w.n * 3 * w.ss * es
    p_bytes = w.n * (w.ss if pinv_diag else 3 * w.ss) * es
    return float(B) * (s_bytes + p_bytes + 3 * w.n * es + 4)


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


# --------------------------------------------------------------------------
# measured HBM traffic (profiles/hbm_traffic.md)
# --------------------------------------------------------------------------

def read_traffic(path=TRAFFIC_FILE):
    """{kernel key: calibrated bytes per dispatch} if the recorded source hash
    matches the current sources, else {}."""
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    m = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel_source_hash():
        return {}
    out = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0] in KERNEL_OF:
            try:
                out[cells[0]] = float(cells[5])
            except ValueError:
                pass
    return out


def _counter_rows(path):
    """(kernel name, counter name, value) per row of a rocprofv3 counter CSV."""
    with open(path, newline="") as f:
        rd = csv.DictReader(f)
        cols = rd.fieldnames or []
        kcol = next(c for c in cols if c.lower() == "kernel_name")
        ncol = next(c for c in cols if c.lower() == "counter_name")
        vcol = next(c for c in cols if c.lower() == "counter_value")
        dcol = next((c for c in cols if c.lower() == "dispatch_id"), None)
        for row in rd:
            yield row[kcol], row[ncol], float(row[vcol]), (row[dcol] if dcol else None)


def _per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} (values of one dispatch summed over
    counter instances)."""
    acc = {}
    for kname, cname, val, did in _counter_rows(path):
        if cname != counter:
            continue
        acc.setdefault((kname, did), 0.0)
        acc[(kname, did)] += val
    out = {}
    for (kname, _), v in acc.items():
        out.setdefault(kname, []).append(v)
    return out


def summarize_pmc(fetch_csv, write_csv, fetch_cmd, write_cmd, out=TRAFFIC_FILE, workloads=None):
    """Calibrated bytes per dispatch for each profiled workload.  workloads
    lists the workloads the profiled command ran (default: all); a kernel
    name that two of them share gets no row, since its counters mix them."""
    keys = list(KERNEL_OF) if workloads is None else list(workloads)
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")

    def find(table, sub):
        hits = [k for k in table if sub in k]
        if len(hits) != 1:
            raise SystemExit("expected one kernel matching %r, found %s" % (sub, hits))
        return float(np.mean(table[hits[0]])), len(table[hits[0]])

    cal_f, _ = find(fetch, "neg_kernel")
    cal_w, _ = find(write, "neg_kernel")
    fr = CALIBRATION_BYTES / (cal_f * 1024.0)
    fw = CALIBRATION_BYTES / (cal_w * 1024.0)
    lines = [
        "# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)",
        "",
        "kernel source sha256: %s" % kernel_source_hash(),
        "",
        "FETCH_SIZE run: `%s`" % fetch_cmd,
        "",
        "WRITE_SIZE run: `%s`" % write_cmd,
        "",
        "Workloads profiled: %s" % ",".join(keys),
        "",
        "Calibration: a negation kernel reading and writing %d bytes reads "
        "FETCH_SIZE = %.1f KiB and WRITE_SIZE = %.1f KiB per dispatch, so "
        "bytes = FETCH_SIZE KiB x 1024 x %.4f + WRITE_SIZE KiB x 1024 x %.4f."
        % (CALIBRATION_BYTES, cal_f, cal_w, fr, fw),
        "",
        "| workload | kernel | dispatches | FETCH_SIZE KiB/dispatch | "
        "WRITE_SIZE KiB/dispatch | calibrated bytes/dispatch |",
        "|---|---|---|---|---|---|",
    ]
    for key in keys:
        sub = KERNEL_OF[key]
        if sum(1 for k2 in keys if KERNEL_OF[k2] == sub) > 1:
            continue
        try:
            f, nd = find(fetch, sub)
            wv, _ = find(write, sub)
        except SystemExit:
            continue
        b = f * 1024.0 * fr + wv * 1024.0 * fw
        lines.append("| %s | %s | %d | %.1f | %.1f | %.0f |" % (key, sub, nd, f, wv, b))
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------

class Timer:
    """HIP events on the stream the library launches on (torch's current
    stream), one before the first and one after the last of the timed
    launches: the average launch duration over the timed region, the short
    gaps between back-to-back launches included.  No events go between the
    launches: on the headline solve a pair around every launch added about
    8 us per step to the wall time and lengthened the launches themselves
    (450 against 442 us)."""

    def __init__(self, torch, steps):
        self.steps = steps
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop(self):
        self.b.record()

    def avg_ms(self):
        return self.a.elapsed_time(self.b) / self.steps


def isolated_ms(torch, fn, reps=10):
    """GPU-side duration per call with the host enqueueing ahead of the GPU
    (a spin kernel holds the stream while the calls are queued), so host
    launch overhead is excluded; measured after the timed region.  fn(k)
    makes call k."""
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for k, (a, b) in enumerate(ev):
        a.record()
        fn(k)
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def roofline(nbytes, avg_ms, traffic, compulsory=None, served_by="hbm"):
    """HBM roofline of a launch.  ``nbytes``: the placement's algorithmic bytes
    (matrices that stay on chip once, re-read ones once per pass).
    ``compulsory``: the bytes any placement must move (matrices once); its
    fraction is reported beside the placement's.  ``served_by``: "hbm" when
    every byte is read once, "hbm+infinity-cache" when the placement re-reads
    a working set that the 256 MB Infinity Cache partly serves (the rate of
    those bytes is then not an HBM rate)."""
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    out = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
           "algorithmic_bytes_per_launch": nbytes, "served_by": served_by}
    if compulsory is not None:
        ca = compulsory / (avg_ms * 1e-3) / 1e9
        out["compulsory_bytes_per_launch"] = compulsory
        out["compulsory_achieved"] = ca
        out["frac_compulsory"] = ca / HBM_PEAK_GBS
    return out


FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X dense fp32 vector
FP64_VECTOR_PEAK_TFLOPS = 78.6


def algorithmic_flops_bdsv(w) -> float:
    """Floating-point operations of one direct solve by the plainest block
    elimination (a multiply-add counts two): per block-row, factor the pivot
    block by Cholesky (2 ss^3 / 3) and solve it for the ss+1 columns of
    [R | y] (2 ss^2 (ss+1)); for every block-row after the first, the update
    [D | b] - L [G | u] (2 ss^2 (ss+1)); the back substitution x_br = u_br -
    G_br x_{br+1} (2 ss^2 per block-row after the last)."""
    ss, kp = w.ss, w.kp
    per_row = 2.0 * ss ** 3 / 3.0 + 2.0 * ss * ss * (ss + 1)
    return kp * per_row + (kp - 1) * (2.0 * ss * ss * (ss + 1) + 2.0 * ss * ss)


# The library is built with packed FP32 instructions disabled, so one fp32
# vector FMA per lane per clock is its ceiling: 256 CUs x 64 FMA/clk x 2 FLOP
# x 2.4 GHz = 78.6 TFLOP/s, half the packed 157.3.
FP32_UNPACKED_PEAK_TFLOPS = 78.6


def roofline_alu(flops, nbytes, avg_ms, traffic, dtype):
    """Arithmetic-bound kernel: useful FLOP/s against the vector peak its
    build can reach (unpacked fp32, or fp64), with the packed fp32 figure and
    the HBM rate of its algorithmic bytes beside it."""
    f32 = np.dtype(dtype) == np.float32
    peak = FP32_UNPACKED_PEAK_TFLOPS if f32 else FP64_VECTOR_PEAK_TFLOPS
    achieved = flops / (avg_ms * 1e-3) / 1e12
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    out = {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
           "frac": achieved / peak, "traffic": traffic,
           "algorithmic_flops_per_launch": flops,
           "algorithmic_bytes_per_launch": nbytes,
           "hbm_achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    if f32:
        out["frac_of_packed_peak"] = achieved / FP32_VECTOR_PEAK_TFLOPS
    return out


def bench_pcg(torch, glass, key, steps, warmup, cpu_budget, with_cpu, traffic,
              cooperative=True):
    cfg = CONFIG_OF[key]
    w = workload_of(key)
    inp = workloads.generate(w)
    dev = torch.device("cuda:0")
    packed = key in PINV_PACKED
    S = torch.from_numpy(inp["S"]).to(dev)
    P = torch.from_numpy(inp["Pinv"]).to(dev)
    if key in UNALIGNED:  # the same values 4 bytes past a 16-byte boundary
        def shifted(t):
            store = torch.empty(t.numel() + 1, dtype=t.dtype, device=dev)
            view = store[1:].view(t.shape)
            view.copy_(t)
            return view
        S, P = shifted(S), shifted(P)
    B = w.n_problems
    if packed:  # the D blocks alone, [B, kp, ss, ss]
        P = P.reshape(B, w.kp, w.ss, 3 * w.ss)[:, :, :, w.ss:2 * w.ss].contiguous()
    b = torch.from_numpy(inp["b"]).to(dev)
    xs = [torch.zeros((B, w.n), dtype=S.dtype, device=dev) for _ in range(steps + warmup)]
    iters = torch.zeros(B, dtype=torch.int32, device=dev)
    status = torch.full((B,), -1, dtype=torch.int32, device=dev)
    grid = w.kind == "grid"
    if grid:
        ws = torch.empty(glass.pcg_grid_workspace_bytes(w.ss, w.kp, S.dtype),
                         dtype=torch.uint8, device=dev)

    # The grid solve is timed with the exclusive launch (this process is the
    # only user of the device); the cooperative launch is timed after it.
    pd = key in PINV_DIAG
    single = key in SINGLE_RED
    if key in NO_HYBRID:
        os.environ["GLASS_AMD_PCG_NO_HYBRID"] = "1"
    else:
        os.environ.pop("GLASS_AMD_PCG_NO_HYBRID", None)
    if key in MULTI:
        os.environ["GLASS_AMD_PCG_MULTI"] = "1"
    else:
        os.environ.pop("GLASS_AMD_PCG_MULTI", None)

    def run(x, exclusive=True):
        if grid:
            glass.pcg_grid(x, S, P, b, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, iters, ws,
                           status, exclusive=exclusive, single_reduction=single,
                           keep_workspace=True)
        else:
            glass.pcg_batched(x, S, P, b, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, iters,
                              status, pinv_block_diagonal=pd, pinv_diagonal_blocks=packed)

    for k in range(warmup):
        run(xs[steps + k])
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    t0 = time.perf_counter()
    tm.start()
    for k in range(steps):
        run(xs[k])
    tm.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    it = iters.cpu().numpy()
    st = status.cpu().numpy()
    avg_ms = tm.avg_ms()
    # S and Pinv count once if they stay on chip (the grid solve and the
    # batched resident placement), else once per pass.
    placement = None if grid else glass.pcg_batched_placement(
        w.ss, w.kp, S.dtype, aligned16=key not in UNALIGNED, pinv_block_diagonal=pd,
        pinv_diagonal_blocks=packed)
    resident = grid or placement in (glass.PLACEMENT_RESIDENT, glass.PLACEMENT_SEVERAL_PER_WAVE) \
        or ("S" if placement == glass.PLACEMENT_S_RESIDENT else False)
    pass_rows = tuple(glass.pcg_batched_pinv_pass_rows(
        w.ss, w.kp, S.dtype, p, aligned16=key not in UNALIGNED, pinv_block_diagonal=pd,
        pinv_diagonal_blocks=packed) for p in (0, 1, 2)) if resident == "S" else None
    nbytes = algorithmic_bytes_pcg(w, it, resident, pinv_diag=pd or packed, pass_rows=pass_rows)
    compulsory = compulsory_bytes_pcg(w, B, pinv_diag=pd or packed)
    served_by = "hbm" if resident is True else "hbm+infinity-cache"
    for k in range(min(10, len(xs))):
        xs[k].zero_()
    iso = isolated_ms(torch, lambda k: run(xs[k]), reps=min(10, len(xs)))
    out = {
        "workload": w.name, "kind": "grid_pcg" if grid else "batched_pcg",
        "kernel": KERNEL_OF[key], "dtype": np.dtype(w.dtype).name, "state_size": w.ss,
        "knot_points": w.kp, "n_problems": B, "solves_per_s": B * steps / wall,
        "ms_per_step": wall * 1e3 / steps, "kernel_ms_avg": avg_ms,
        "kernel_ms_isolated": iso,
        "iterations": {str(k): int(v) for k, v in zip(*np.unique(it, return_counts=True))},
        # every timed solve must have converged (a breakdown or a grid
        # timeout would otherwise be timed as a fast valid solve)
        "not_converged": int((st != glass.CONVERGED).sum()),
        "valid": bool(np.all(st == glass.CONVERGED)),
        "roofline": roofline(nbytes, avg_ms, traffic.get(key), compulsory, served_by),
    }
    if not grid:
        out["us_per_iteration"] = avg_ms * 1e3 / max(1, int(it.max()))
    if grid:
        out["launch"] = "exclusive"
        out["workspace"] = "kept (GLASS_GRID_KEEP_WORKSPACE: no per-solve clearing kernel)"
        out["us_per_iteration"] = avg_ms * 1e3 / max(1, int(it[0]))
        if cooperative:
            for k in range(min(10, len(xs))):
                xs[k].zero_()
            out["kernel_ms_isolated_cooperative"] = isolated_ms(
                torch, lambda k: run(xs[k], exclusive=False), reps=min(10, len(xs)))
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


def bench_bdmv(torch, glass, steps, warmup, cpu_budget, with_cpu, traffic):
    w = workloads.WORKLOADS[1]
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
    tm.start()
    for k in range(steps):
        glass.bdmv_batched(y, S, v, w.ss, w.kp)
    tm.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = tm.avg_ms()
    nbytes = algorithmic_bytes_bdmv(w, w.n_problems)
    iso = isolated_ms(torch, lambda k: glass.bdmv_batched(y, S, v, w.ss, w.kp))
    out = {
        "workload": w.name, "kind": "bdmv", "kernel": KERNEL_OF["bdmv1"], "dtype": "float32",
        "state_size": w.ss, "knot_points": w.kp, "n_problems": w.n_problems,
        "gb_per_s": nbytes / (wall / steps) / 1e9, "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_avg": avg_ms,
        "kernel_ms_isolated": iso,
        "roofline": roofline(nbytes, avg_ms, traffic.get("bdmv1")),
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


def bench_bdsv(torch, glass, key, steps, warmup, cpu_budget, with_cpu, traffic):
    w = workload_of(key)
    inp = workloads.generate(w, with_pinv=False)
    dev = torch.device("cuda:0")
    S = torch.from_numpy(inp["S"]).to(dev)
    b = torch.from_numpy(inp["b"]).to(dev)
    B = w.n_problems
    x = torch.zeros((B, w.n), dtype=S.dtype, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    # The per-block-row factors go to a workspace in HBM (more problems per CU).
    ws = torch.empty(glass.bdsv_workspace_bytes(w.ss, w.kp, B, S.dtype), dtype=torch.uint8,
                     device=dev)
    for _ in range(warmup):
        glass.bdsv_batched(x, S, b, w.ss, w.kp, status, workspace=ws)
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    t0 = time.perf_counter()
    tm.start()
    for k in range(steps):
        glass.bdsv_batched(x, S, b, w.ss, w.kp, status, workspace=ws)
    tm.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = tm.avg_ms()
    iso = isolated_ms(torch, lambda k: glass.bdsv_batched(x, S, b, w.ss, w.kp, status,
                                                         workspace=ws))
    es = np.dtype(w.dtype).itemsize
    # S once, b read, x written, status; plus the factors [G|u] written to and
    # read back from the workspace (kp*ss*(ss+1) each way)
    nbytes = float(B) * (w.n * 3 * w.ss * es + 2 * w.n * es + 4
                         + 2 * w.kp * w.ss * (w.ss + 1) * es)
    out = {
        "workload": "bdsv_ss14_kp32_b4096_f32", "kind": "bdsv", "kernel": KERNEL_OF[key],
        "dtype": np.dtype(w.dtype).name, "state_size": w.ss, "knot_points": w.kp,
        "n_problems": B, "solves_per_s": B * steps / wall, "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_avg": avg_ms,
        "kernel_ms_isolated": iso,
        "not_spd": int((status.cpu().numpy() != 0).sum()),
        "roofline": roofline_alu(B * algorithmic_flops_bdsv(w), nbytes, avg_ms, traffic.get(key),
                                 w.dtype),
    }
    if with_cpu:
        import oracle
        nt = cpu_threads()
        sec, calls = time_cpu(lambda: oracle.bdsv(inp["S"], inp["b"], w.ss, w.kp, "f32", nt),
                              cpu_budget)
        out["cpu_baseline"] = {"value": B / sec, "unit": "solves/s", "cores": nt, "kind": "oracle",
                               "sample": "the full %d-problem workload, %d repetitions" % (B, calls)}
    return out


def measured_read_gbs(torch, glass, nbytes=1 << 30, reps=10):
    """The device's streaming-read rate: glass_stream_read over 1 GiB (read
    once with coalesced 16-byte non-temporal loads; median of 10).  The HBM
    fractions are also given against it: it is the practical ceiling of a
    read-bound kernel, which the vendor peak is not.  The checksum of the
    read is verified."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    for _ in range(3):
        glass.stream_read(src, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        glass.stream_read(src, sink)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    # 2^28 words of 1: each read buffer XORs to 0 (an even number of 1s).
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy())) == 0
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9


def measured_lds_gbs(torch, glass, rounds=2048, reps=10, width=16):
    """The device's LDS read rate: glass_lds_read (loads of ``width`` bytes
    per lane by every thread of 8 workgroups per compute unit; median of 10),
    in GB/s.  The LDS-side fractions of the placements that stream through
    LDS are priced against the 16-byte rate.  Every workgroup's checksum must
    agree."""
    dev = torch.device("cuda:0")
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    wg = glass.lds_read(sink, rounds, width)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        glass.lds_read(sink, rounds, width)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    words = sink[:wg].cpu().numpy()
    assert np.all(words == words[0])
    return wg * 256 * rounds * 8 * 16 / (ms * 1e-3) / 1e9


def torch_copy_gbs(torch, nbytes=1 << 30, reps=10):
    """Device-to-device torch copy of 1 GiB (read + write bytes per second),
    reported for context."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def calibration_copy(torch):
    """A plain streaming kernel of known traffic: y = -x over 1 GiB (reads
    1 GiB, writes 1 GiB).  Its counters calibrate FETCH_SIZE / WRITE_SIZE."""
    dev = torch.device("cuda:0")
    x = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="all",
                    help="comma list of %s or 'all'" % ",".join(CONFIG_OF))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-budget", type=float, default=4.0,
                    help="seconds of oracle time per workload baseline")
    ap.add_argument("--calibration-copy", action="store_true")
    ap.add_argument("--no-cooperative", action="store_true",
                    help="skip timing the grid solve's cooperative launch (for profiler runs: "
                         "rocprofv3 ends with a segmentation fault at process exit after "
                         "cooperative launches)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--pmc-commands", nargs=2, default=("?", "?"),
                    metavar=("FETCH_CMD", "WRITE_CMD"))
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], *args.pmc_commands,
                      workloads=None if args.workloads == "all" else
                      [s.strip() for s in args.workloads.split(",") if s.strip()])
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the batched "
              "problems are independent, so a batch would be split across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_tridiagonal_pcg_bdmv_amd as glass
    # Some rows select a placement through the library's GLASS_AMD_* switches
    # (pcg3_stream, the several-per-wave rows), which it honours only in a
    # process that sets this before its first call.
    os.environ["GLASS_AMD_TUNING"] = "1"
    glass.load()
    torch.cuda.set_device(0)

    sel = list(CONFIG_OF) if args.workloads == "all" else \
        [s.strip() for s in args.workloads.split(",") if s.strip()]
    with_cpu = not args.no_cpu
    traffic = read_traffic()
    res = {}
    for name in sel:
        print("[bench] %s ..." % name, file=sys.stderr, flush=True)
        if name == "bdmv1":
            res[name] = bench_bdmv(torch, glass, args.steps, args.warmup, args.cpu_budget,
                                   with_cpu, traffic)
        elif name == "bdsv2":
            res[name] = bench_bdsv(torch, glass, name, args.steps, args.warmup, args.cpu_budget,
                                   with_cpu, traffic)
        else:
            # the headline workload gets the larger CPU budget (10 s)
            budget = max(args.cpu_budget, 10.0) if name == "pcg3" else args.cpu_budget
            # pcg3_stream runs pcg3's inputs in another placement: no second
            # CPU baseline
            res[name] = bench_pcg(torch, glass, name, args.steps, args.warmup, budget,
                                  with_cpu and name not in NO_HYBRID | MULTI | UNALIGNED, traffic,
                                  cooperative=not args.no_cooperative)
        print("[bench] %s done: %s" % (name, json.dumps(res[name])[:300]), file=sys.stderr,
              flush=True)
    if args.calibration_copy:
        calibration_copy(torch)
    read_gbs = measured_read_gbs(torch, glass)
    lds_gbs = {w: measured_lds_gbs(torch, glass, width=w) for w in (16, 8, 4)}
    copy_gbs = torch_copy_gbs(torch)
    for r in res.values():
        rl = r["roofline"]
        gbs = rl["achieved"] if rl["bound"] == "hbm" else rl.get("hbm_achieved_gbs")
        if gbs is not None:
            rl["frac_of_measured_read"] = gbs / read_gbs
        if rl.get("compulsory_achieved") is not None:
            rl["frac_compulsory_of_measured_read"] = rl["compulsory_achieved"] / read_gbs

    head = res.get("pcg3") or next(iter(res.values()))
    w = workloads.WORKLOADS[3]
    line = {
        "metric": METRIC,
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
        "measured_read_gbs": read_gbs,
        "measured_lds_gbs": lds_gbs[16],
        "measured_lds_gbs_by_load_width": {"%d B" % w: v for w, v in lds_gbs.items()},
        "torch_copy_gbs": copy_gbs,
        "workloads": res,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
