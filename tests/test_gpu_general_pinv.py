"""GPU parity with a general block-tridiagonal preconditioner (non-zero L and
R blocks; GLASS user guide, page "Block-tridiagonal Solves", section
"Solve -- glass::pcg": Pinv is a block-tridiagonal matrix in [L|D|R] form).

The preconditioner is the generator's ``pinv="tridiagonal"`` option, the SPD
first-order approximation D^-1 - D^-1 E D^-1 of S^-1.  Every placement that
reads Pinv's L/R columns is run on it: the S-resident placement with and
without chunks pinned on chip (in LDS, and in the registers of waves without
a last S chunk), the streamed placements with and without prefetch, the
register-resident placement at 1-4 rows per lane, the generic state sizes,
and both forms of the grid solve (whose neighbour r and ghost p rows feed
Pinv's L/R blocks at the partition edges) at several grid sizes, including
partitions of two block-rows.  Placements of the batched solve give the same
bits; each result meets the oracle bars of gpu_common.  Long solves (about
30-80 iterations) run on a stiffer system with Pinv = I and with the
tridiagonal Pinv."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads
from gpu_common import assert_pcg_parity, pcg_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def tri_inputs(cfg, n_problems=None, dtype=None):
    w = replace(workloads.WORKLOADS[cfg], pinv="tridiagonal")
    if dtype is not None:
        w = replace(w, dtype=dtype)
    return w, workloads.generate(w, n_problems=n_problems)


def random_tri_inputs(ss, kp, B, margin, dtype, seed, x0_random=False):
    rng = np.random.default_rng(seed)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, margin)
    P = workloads.block_tridiagonal_pinv(S, D, dtype)
    b = rng.standard_normal((B, kp * ss)).astype(dtype)
    x0 = rng.standard_normal((B, kp * ss)).astype(dtype) if x0_random else \
        np.zeros((B, kp * ss), dtype)
    return {"S": S.astype(dtype), "Pinv": P, "b": b, "x0": x0}


def assert_same(ref, got, what):
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v, err_msg=what)


# (name, environment) of the placements an [L|D|R] Pinv can take for the
# specialised S-resident sizes, in the order they are run.
S_RESIDENT_PLACEMENTS = [
    ("S resident, chunks pinned", {}),
    ("S resident, nothing pinned", {"GLASS_AMD_PCG_NO_PIN": "1"}),
    ("streamed with prefetch", {"GLASS_AMD_PCG_NO_HYBRID": "1"}),
    ("streamed, plain staging", {"GLASS_AMD_PCG_NO_HYBRID": "1",
                                 "GLASS_AMD_PCG_NO_PREFETCH": "1"}),
]


def run_placements(gpu, monkeypatch, inp, ss, kp, max_iters, rel, abs_tol, placements):
    out = []
    for name, env in placements:
        for k in ("GLASS_AMD_PCG_NO_PIN", "GLASS_AMD_PCG_NO_HYBRID", "GLASS_AMD_PCG_NO_PREFETCH",
                  "GLASS_AMD_PCG_STREAMED", "GLASS_AMD_PCG_RPT", "GLASS_AMD_PCG_RES_RPT"):
            monkeypatch.delenv(k, raising=False)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        say("  %s" % name)
        out.append((name, pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)))
    for k in ("GLASS_AMD_PCG_NO_PIN", "GLASS_AMD_PCG_NO_HYBRID", "GLASS_AMD_PCG_NO_PREFETCH",
              "GLASS_AMD_PCG_STREAMED", "GLASS_AMD_PCG_RPT", "GLASS_AMD_PCG_RES_RPT"):
        monkeypatch.delenv(k, raising=False)
    return out


def test_general_pinv_headline_workload_every_placement(gpu, monkeypatch):
    """The ss=21 kp=64 workload, all 2048 problems, with the tridiagonal Pinv:
    S-resident with 4 of 21 Pinv chunks pinned (wave 0's last chunk in LDS,
    waves 5-7's chunk 0 in registers), without pinning, streamed with
    prefetch and plain; bit-identical, and the oracle bars."""
    w, inp = tri_inputs(3)
    assert gpu.pcg_batched_pinned_rows(w.ss, w.kp, torch.float32) == 256
    assert gpu.pcg_batched_placement(w.ss, w.kp, torch.float32) == gpu.PLACEMENT_S_RESIDENT
    say("pcg cfg3 full, block-tridiagonal Pinv")
    runs = run_placements(gpu, monkeypatch, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                          S_RESIDENT_PLACEMENTS)
    ref = runs[0][1]
    assert np.all(ref[2] == gpu.CONVERGED)
    for name, got in runs[1:]:
        assert_same(ref, got, name)
    its = assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, ref, np.float32)
    say("  iterations: %s" % dict(zip(*np.unique(its, return_counts=True))))


@pytest.mark.parametrize("ss,kp,B,dtype", [
    (21, 40, 9, np.float32),    # 14 chunks, 2 per wave: LDS slot + register-held chunks
    (21, 60, 5, np.float32),    # 20 chunks, ragged last
    (21, 52, 4, np.float32),    # 18 chunks on 6-7 waves, ragged
    (21, 20, 4, np.float32),    # one row per lane
    (21, 4, 3, np.float32),     # two chunks, the second ragged
    (14, 32, 24, np.float64),   # the ss=14 systems in float64 (S resident)
    (12, 70, 3, np.float64),    # 14 chunks, two rows per lane
])
def test_general_pinv_s_resident_shapes(gpu, monkeypatch, ss, kp, B, dtype):
    inp = random_tri_inputs(ss, kp, B, 0.1, dtype, seed=ss * 1000 + kp, x0_random=True)
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    assert gpu.pcg_batched_placement(ss, kp, tdt) == gpu.PLACEMENT_S_RESIDENT
    rel = 1e-8 if dtype == np.float32 else 1e-14
    say("pcg ss=%d kp=%d B=%d %s block-tridiagonal Pinv (pinned rows %d)"
        % (ss, kp, B, np.dtype(dtype).name, gpu.pcg_batched_pinned_rows(ss, kp, tdt)))
    runs = run_placements(gpu, monkeypatch, inp, ss, kp, 300, rel, 0.0, S_RESIDENT_PLACEMENTS)
    ref = runs[0][1]
    assert np.all(ref[2] == gpu.CONVERGED)
    for name, got in runs[1:]:
        assert_same(ref, got, name)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, ref, dtype)


def test_general_pinv_resident_workload_full_and_streamed(gpu, monkeypatch):
    """The ss=14 kp=32 workload, all 4096 problems, with the tridiagonal Pinv
    in the register-resident placement (one and two rows per lane), then a
    subset through the streamed placements at 1, 2, 3, 4 and 8 rows per
    lane, with and without prefetch: the same bits, and the oracle bars."""
    w, inp = tri_inputs(2)
    assert gpu.pcg_batched_placement(w.ss, w.kp, torch.float32) == gpu.PLACEMENT_RESIDENT
    say("pcg cfg2 full, block-tridiagonal Pinv")
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    assert np.all(ref[2] == gpu.CONVERGED)
    its = assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, ref, np.float32)
    say("  iterations: %s" % dict(zip(*np.unique(its, return_counts=True))))
    monkeypatch.setenv("GLASS_AMD_PCG_RES_RPT", "2")
    say("  resident, two rows per lane")
    assert_same(ref, pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol),
                "resident rows/lane=2")
    monkeypatch.delenv("GLASS_AMD_PCG_RES_RPT")
    sub = {k: v[:24] for k, v in inp.items()}
    ref24 = tuple(a[:24] for a in ref)
    monkeypatch.setenv("GLASS_AMD_PCG_STREAMED", "1")
    for rpt in ("1", "2", "3", "4", "8"):
        for pf in ("0", "1"):
            monkeypatch.setenv("GLASS_AMD_PCG_RPT", rpt)
            if pf == "0":
                monkeypatch.setenv("GLASS_AMD_PCG_NO_PREFETCH", "1")
            else:
                monkeypatch.delenv("GLASS_AMD_PCG_NO_PREFETCH", raising=False)
            say("  streamed rows/lane=%s prefetch=%s" % (rpt, pf))
            got = pcg_gpu(gpu, sub, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
            assert_same(ref24, got, "streamed rpt=%s pf=%s" % (rpt, pf))


@pytest.mark.parametrize("rpt", ["1", "2", "3", "4"])
def test_general_pinv_small_workload_rows_per_lane(gpu, monkeypatch, rpt):
    """The ss=6 kp=32 workload (64 problems) with the tridiagonal Pinv at 1-4
    resident rows per lane (3 is one wave per problem): the same bits, and
    the oracle bars."""
    w, inp = tri_inputs(0)
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    monkeypatch.setenv("GLASS_AMD_PCG_RES_RPT", rpt)
    say("pcg cfg0 block-tridiagonal Pinv, resident rows/lane=%s" % rpt)
    got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    assert_same(ref, got, "rows/lane=%s" % rpt)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)


@pytest.mark.parametrize("ss,kp,B,dtype", [
    (9, 23, 5, np.float32),     # runtime state size, ragged chunk, element paths
    (9, 32, 5, np.float32),     # runtime state size, 16-byte paths
    (33, 10, 3, np.float32),
    (64, 5, 2, np.float32),
    (1, 300, 3, np.float32),
    (6, 200, 2, np.float64),    # streamed specialised size, float64
    (21, 100, 2, np.float32),   # 2100 rows
    (7, 150, 3, np.float64),
])
def test_general_pinv_other_shapes(gpu, ss, kp, B, dtype):
    inp = random_tri_inputs(ss, kp, B, 0.2, dtype, seed=ss * 77 + kp, x0_random=True)
    rel = 1e-8 if dtype == np.float32 else 1e-14
    say("pcg ss=%d kp=%d B=%d %s block-tridiagonal Pinv" % (ss, kp, B, np.dtype(dtype).name))
    res = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
    assert np.all(res[2] == gpu.CONVERGED)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, res, dtype)


# ---------------------------------------------------------------------------
# grid solve
# ---------------------------------------------------------------------------

@pytest.fixture(params=["standard", "single"])
def variant(request):
    return request.param == "single"


def grid_gpu(glass, inp, ss, kp, max_iters, rel_tol, abs_tol, exclusive=False, single=False):
    t = {k: to_dev(v) for k, v in inp.items()}
    x = t["x0"].clone()
    iters = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros(2, dtype=x.dtype, device="cuda")
    ws = torch.empty(glass.pcg_grid_workspace_bytes(ss, kp, x.dtype), dtype=torch.uint8,
                     device="cuda")
    glass.pcg_grid(x, t["S"], t["Pinv"], t["b"], ss, kp, max_iters, rel_tol, abs_tol,
                   iters, ws, status, rho, exclusive=exclusive, single_reduction=single)
    torch.cuda.synchronize()
    return (x.cpu().numpy(), iters.cpu().numpy(), status.cpu().numpy(),
            rho.cpu().numpy().reshape(1, 2))


def test_grid_general_pinv_full_chain(gpu, variant):
    """The kp=8192 ss=12 fp64 chain with the tridiagonal Pinv, every entry of
    x checked; the exclusive launch gives the same bits."""
    w, inp = tri_inputs(4)
    say("grid ss=12 kp=8192 fp64 block-tridiagonal Pinv single=%s" % variant)
    res = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=variant)
    assert res[2][0] == gpu.CONVERGED, res[2]
    its = assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, res, np.float64)
    say("  iterations: %d" % its[0])
    excl = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, exclusive=True,
                    single=variant)
    assert_same(res, excl, "exclusive launch")


@pytest.mark.parametrize("wgs", [2, 24, 512])
def test_grid_general_pinv_partitions(gpu, monkeypatch, wgs, variant):
    """kp=1024 ss=12 fp64 at 2, 24 and 512 workgroups (512: every partition
    is two block-rows, so each workgroup's edges are all its rows)."""
    inp = random_tri_inputs(12, 1024, 1, 0.05, np.float64, seed=91, x0_random=True)
    monkeypatch.setenv("GLASS_AMD_GRID_WGS", str(wgs))
    say("grid kp=1024 wgs=%d block-tridiagonal Pinv single=%s" % (wgs, variant))
    res = grid_gpu(gpu, inp, 12, 1024, 300, 1e-12, 0.0, single=variant)
    assert res[2][0] == gpu.CONVERGED
    assert_pcg_parity(inp, 12, 1024, 300, 1e-12, 0.0, res, np.float64)


@pytest.mark.parametrize("ss,kp,dtype", [(6, 300, np.float32), (14, 97, np.float32),
                                         (21, 40, np.float32), (5, 33, np.float64),
                                         (3, 4, np.float64), (12, 8192, np.float32)])
def test_grid_general_pinv_shapes(gpu, ss, kp, dtype, variant):
    inp = random_tri_inputs(ss, kp, 1, 0.1, dtype, seed=ss * 13 + kp)
    rel = 1e-7 if dtype == np.float32 else 1e-12
    say("grid ss=%d kp=%d %s block-tridiagonal Pinv single=%s"
        % (ss, kp, np.dtype(dtype).name, variant))
    res = grid_gpu(gpu, inp, ss, kp, 500, rel, 0.0, single=variant)
    assert res[2][0] == gpu.CONVERGED
    assert_pcg_parity(inp, ss, kp, 500, rel, 0.0, res, dtype)


# ---------------------------------------------------------------------------
# long solves
# ---------------------------------------------------------------------------

def stiff_inputs(ss, kp, B, dtype, pinv, seed):
    """A stiffer system (generator strips scaled by 0.01 plus the block 1-D
    Laplacian) with Pinv = I or the tridiagonal preconditioner."""
    rng = np.random.default_rng(seed)
    S0, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.01)
    S = workloads.laplacian_coupled_strips(S0, 0.01)
    D = np.ascontiguousarray(S[:, :, :, ss:2 * ss])
    P = workloads.identity_pinv(B, ss, kp) if pinv == "identity" else \
        workloads.block_tridiagonal_pinv(S, D)
    return {"S": S.astype(dtype), "Pinv": P.astype(dtype),
            "b": rng.standard_normal((B, kp * ss)).astype(dtype),
            "x0": np.zeros((B, kp * ss), dtype)}


@pytest.mark.parametrize("ss,kp,B,dtype,pinv", [
    (14, 32, 16, np.float64, "identity"),     # about 70 iterations, resident placement
    (21, 64, 4, np.float64, "identity"),      # streamed (float64 ss=21)
    (21, 64, 8, np.float32, "tridiagonal"),   # S resident, float32
    (6, 32, 8, np.float32, "identity"),
])
def test_long_batched_solves(gpu, ss, kp, B, dtype, pinv):
    inp = stiff_inputs(ss, kp, B, dtype, pinv, seed=ss + kp)
    rel = 1e-20 if dtype == np.float64 else 1e-10
    say("pcg long solve ss=%d kp=%d %s Pinv=%s" % (ss, kp, np.dtype(dtype).name, pinv))
    res = pcg_gpu(gpu, inp, ss, kp, 2000, rel, 0.0)
    assert np.all(res[2] == gpu.CONVERGED)
    its = assert_pcg_parity(inp, ss, kp, 2000, rel, 0.0, res, dtype)
    say("  iterations %d-%d" % (its.min(), its.max()))
    assert its.min() >= 15


@pytest.mark.parametrize("pinv", ["identity", "tridiagonal"])
def test_long_grid_solve(gpu, pinv, variant):
    inp = stiff_inputs(12, 2048, 1, np.float64, pinv, seed=17)
    say("grid long solve kp=2048 fp64 Pinv=%s single=%s" % (pinv, variant))
    res = grid_gpu(gpu, inp, 12, 2048, 2000, 1e-20, 0.0, single=variant)
    assert res[2][0] == gpu.CONVERGED
    its = assert_pcg_parity(inp, 12, 2048, 2000, 1e-20, 0.0, res, np.float64)
    say("  iterations %d" % its[0])
    assert its[0] >= 15


def test_s_resident_random_shapes_match_streamed(gpu, monkeypatch):
    """Seeded random shapes in the S-resident placement (ss = 12, 14, 21;
    fp32 and fp64; kp up to the placement's limit, so ragged last chunks,
    pinned and register-held chunks and odd/even carried-chunk patterns all
    occur; both preconditioners; zero and random x0): bit for bit the
    streamed placement's results, and the oracle bar on the first cases."""
    rng = np.random.default_rng(20261203)
    shapes = [(21, np.float32, 73), (14, np.float64, 56), (12, np.float64, 82)]
    seen = 0
    for case in range(24):
        ss, dtype, kmax = shapes[case % 3]
        kp = int(rng.integers(1, kmax + 1))
        B = int(rng.integers(1, 97))
        tdt = torch.float32 if dtype == np.float32 else torch.float64
        monkeypatch.delenv("GLASS_AMD_PCG_NO_HYBRID", raising=False)
        assert gpu.pcg_batched_placement(ss, kp, tdt) == gpu.PLACEMENT_S_RESIDENT, (ss, kp)
        r2 = np.random.default_rng(int(rng.integers(0, 1 << 30)))
        S, D = workloads.random_spd_strips(r2, B, ss, kp, 0.1)
        P = workloads.block_tridiagonal_pinv(S, D, dtype) if case % 2 else \
            workloads.block_jacobi_pinv(D, dtype)
        inp = {"S": S.astype(dtype), "Pinv": P,
               "b": r2.standard_normal((B, kp * ss)).astype(dtype),
               "x0": (r2.standard_normal((B, kp * ss)) if case % 4 == 3
                      else np.zeros((B, kp * ss))).astype(dtype)}
        rel = 1e-6 if dtype == np.float32 else 1e-12
        say("S-resident random shape %d: ss=%d kp=%d B=%d %s, Pinv rows per pass %s" % (
            case, ss, kp, B, np.dtype(dtype).name,
            [gpu.pcg_batched_pinv_pass_rows(ss, kp, tdt, p) for p in (0, 1, 2)]))
        got = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
        monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
        ref = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
        for u, v in zip(got, ref):
            np.testing.assert_array_equal(u, v)
        if case < 6:
            assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, got, dtype)
        seen += 1
    assert seen == 24


def test_register_held_pinv_chunk_staged_or_direct(gpu, monkeypatch):
    """The waves that keep Pinv's chunk 0 in registers load it through their
    LDS stage after their S chunks (default) or row by row
    (GLASS_AMD_PCG_PREG_STAGE=0): the same values in the same registers, so
    the ss=21 kp=64 workload gives the same bits either way."""
    w = replace(workloads.WORKLOADS[3], pinv="tridiagonal")
    inp = workloads.generate(w, n_problems=256)
    say("ss=21 kp=64 register-held Pinv chunk: staged vs row by row")
    got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    monkeypatch.setenv("GLASS_AMD_PCG_PREG_STAGE", "0")
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    for u, v in zip(got, ref):
        np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)
