"""GPU parity of glass_pcg_grid (one chain over a cooperative grid) against
the CPU oracle through the C ABI: iterations within +-2, x within 1e-10
(fp64) / 1e-4 (fp32) relative L2 of the float64 oracle at the same
iteration count, final criterion met."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import X_REL, assert_pcg_parity, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["standard", "single"])
def variant(request):
    """The standard steps (two grid reductions per iteration) or the
    single-reduction form (GLASS_GRID_SINGLE_REDUCTION); both are held to
    the same oracle bar."""
    return request.param == "single"


def grid_gpu(glass, inp, ss, kp, max_iters, rel_tol, abs_tol, exclusive=False, single=False):
    t = {k: to_dev(v) for k, v in inp.items()}
    x = t["x0"].clone()
    iters = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros(2, dtype=x.dtype, device="cuda")
    nbytes = glass.pcg_grid_workspace_bytes(ss, kp, x.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    glass.pcg_grid(x, t["S"], t["Pinv"], t["b"], ss, kp, max_iters, rel_tol, abs_tol,
                   iters, ws, status, rho, exclusive=exclusive, single_reduction=single)
    torch.cuda.synchronize()
    return (x.cpu().numpy(), iters.cpu().numpy(), status.cpu().numpy(),
            rho.cpu().numpy().reshape(1, 2))


def test_grid_full_chain_fp64(gpu, variant):
    """The kp=8192, ss=12 fp64 chain, every entry of x checked."""
    w = workloads.WORKLOADS[4]
    inp = workloads.generate(w)
    say("grid ss=12 kp=8192 fp64 single=%s" % variant)
    res = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=variant)
    assert res[2][0] == gpu.CONVERGED, res[2]
    its = assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, res, np.float64)
    say("  iterations: %d" % its[0])


@pytest.mark.parametrize("ss,kp,dtype", [(12, 64, np.float64), (6, 300, np.float32),
                                         (14, 97, np.float32), (21, 40, np.float32),
                                         (5, 33, np.float64), (3, 4, np.float64),
                                         (12, 5000, np.float32), (6, 300, np.float64),
                                         (14, 97, np.float64)])
def test_grid_matches_oracle_and_batched(gpu, ss, kp, dtype, variant):
    """Specialised and runtime state sizes, partitions of uneven length, the
    minimum chain (kp = 4).  Also cross-checked with the batched solve of the
    same single problem.  fp64 at ss = 6, 12, 14 and fp32 at ss = 12 have
    blocks of whole 16-byte vectors, read with 16-byte LDS loads."""
    rng = np.random.default_rng(ss * 7 + kp)
    S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.1, dtype)
    inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
           "b": rng.standard_normal((1, kp * ss)).astype(dtype),
           "x0": np.zeros((1, kp * ss), dtype)}
    rel = 1e-10 if dtype == np.float64 else 1e-7
    say("grid ss=%d kp=%d %s single=%s" % (ss, kp, np.dtype(dtype).name, variant))
    res = grid_gpu(gpu, inp, ss, kp, 500, rel, 0.0, single=variant)
    assert res[2][0] == gpu.CONVERGED
    assert_pcg_parity(inp, ss, kp, 500, rel, 0.0, res, dtype)
    if kp * ss <= 8192:
        from gpu_common import pcg_gpu
        bat = pcg_gpu(gpu, inp, ss, kp, 500, rel, 0.0)
        assert abs(int(bat[1][0]) - int(res[1][0])) <= 2
        num = np.linalg.norm(bat[0][0].astype(np.float64) - res[0][0])
        den = np.linalg.norm(bat[0][0].astype(np.float64))
        if bat[1][0] == res[1][0]:
            assert num / den <= X_REL[dtype]


@pytest.mark.parametrize("wgs", [2, 8, 24, 64, 512])
def test_grid_partition_count_does_not_change_the_answer(gpu, monkeypatch, wgs, variant):
    """Different grid sizes change only the summation tree of the dots."""
    rng = np.random.default_rng(77)
    ss, kp = 12, 2048
    S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.05, np.float64)
    inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D), "b": rng.standard_normal((1, kp * ss)),
           "x0": np.zeros((1, kp * ss))}
    monkeypatch.setenv("GLASS_AMD_GRID_WGS", str(wgs))
    say("grid wgs=%d single=%s" % (wgs, variant))
    res = grid_gpu(gpu, inp, ss, kp, 200, 1e-10, 0.0, single=variant)
    assert res[2][0] == gpu.CONVERGED
    assert_pcg_parity(inp, ss, kp, 200, 1e-10, 0.0, res, np.float64)


def test_grid_status_cases(gpu, variant):
    rng = np.random.default_rng(5)
    ss, kp = 6, 64
    S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.3, np.float64)
    P = workloads.block_jacobi_pinv(D)
    b = rng.standard_normal((1, kp * ss))
    x0 = rng.standard_normal((1, kp * ss))
    base = {"S": S, "Pinv": P, "b": b, "x0": x0}
    say("grid max_iters=3 single=%s" % variant)
    x, it, st, _ = grid_gpu(gpu, base, ss, kp, 3, 1e-12, 0.0, single=variant)
    assert it[0] == 3 and st[0] == gpu.MAX_ITERS
    xo, _, _, _ = oracle.pcg(x0, S, P, b, ss, kp, 3, 1e-12, 0.0, "f64")
    assert np.linalg.norm(x - xo) <= 1e-10 * np.linalg.norm(xo)
    say("grid breakdown")
    x, it, st, _ = grid_gpu(gpu, dict(base, S=-S), ss, kp, 20, 1e-8, 0.0, single=variant)
    assert st[0] == gpu.BREAKDOWN and it[0] == 0
    np.testing.assert_array_equal(x, x0)
    say("grid b=0, x0=0")
    x, it, st, _ = grid_gpu(gpu, dict(base, b=0 * b, x0=0 * x0), ss, kp, 20, 1e-8, 0.0,
                            single=variant)
    assert st[0] == gpu.CONVERGED and it[0] == 0 and np.all(x == 0)


def test_grid_full_chain_fp32_variant(gpu, variant):
    """The float32 variant of the kp=8192 chain as bench.py times it
    (rel_tol 1e-7), every entry of x checked."""
    from dataclasses import replace
    w = replace(workloads.WORKLOADS[4], dtype=np.float32, rel_tol=1e-7)
    inp = workloads.generate(w)
    say("grid ss=12 kp=8192 fp32 single=%s" % variant)
    res = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=variant)
    assert res[2][0] == gpu.CONVERGED, res[2]
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, res, np.float32)


@pytest.mark.parametrize("ss,kp,dtype", [(12, 8192, np.float64), (12, 8192, np.float32),
                                         (21, 40, np.float32), (5, 33, np.float64)])
def test_grid_exclusive_launch_is_bit_identical(gpu, ss, kp, dtype):
    """GLASS_GRID_EXCLUSIVE changes only how the grid is dispatched: x,
    iterations, status and rho match the cooperative launch bit for bit,
    also on two solves in a row that reuse the workspace."""
    if kp == 8192:
        from dataclasses import replace
        w = replace(workloads.WORKLOADS[4], dtype=dtype,
                    rel_tol=1e-7 if dtype == np.float32 else workloads.WORKLOADS[4].rel_tol)
        inp = workloads.generate(w)
        rel = w.rel_tol
    else:
        rng = np.random.default_rng(ss * 11 + kp)
        S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.1, dtype)
        inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
               "b": rng.standard_normal((1, kp * ss)).astype(dtype),
               "x0": np.zeros((1, kp * ss), dtype)}
        rel = 1e-10 if dtype == np.float64 else 1e-7
    say("grid exclusive ss=%d kp=%d %s" % (ss, kp, np.dtype(dtype).name))
    coop = grid_gpu(gpu, inp, ss, kp, 500, rel, 0.0)
    for _ in range(2):
        excl = grid_gpu(gpu, inp, ss, kp, 500, rel, 0.0, exclusive=True)
        assert excl[2][0] == gpu.CONVERGED
        for a, b in zip(coop, excl):
            np.testing.assert_array_equal(a, b)


def test_grid_single_reduction_agrees_with_standard_and_repeats(gpu):
    """The single-reduction form against the standard steps on the fp64
    chain: the same iteration count and status, x within 1e-12 relative
    (rounding only), rho_init equal to rounding; and bit-identical repeats,
    also with the exclusive launch."""
    w = workloads.WORKLOADS[4]
    inp = workloads.generate(w)
    say("grid single vs standard fp64")
    std = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    one = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=True)
    assert one[1][0] == std[1][0] and one[2][0] == std[2][0]
    rel = np.linalg.norm(one[0] - std[0]) / np.linalg.norm(std[0])
    assert rel <= 1e-12, rel
    np.testing.assert_allclose(one[3][0, 0], std[3][0, 0], rtol=1e-12)
    again = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=True,
                     exclusive=True)
    for u, v in zip(one, again):
        np.testing.assert_array_equal(u, v)


def test_grid_timeout_path_reports_and_drains(gpu, monkeypatch, variant):
    """The bounded-poll path, forced from the host: with a spin limit of 0
    the first poll that finds a partial missing gives up (workgroups reach
    the first barrier microseconds apart after their row loads).  The solve
    reports GLASS_PCG_GRID_TIMEOUT, every workgroup leaves (the call
    returns), and the next solve on the same workspace is normal."""
    w = workloads.WORKLOADS[4]
    inp = workloads.generate(w)
    monkeypatch.setenv("GLASS_AMD_GRID_SPIN_LIMIT", "0")
    say("grid forced timeout single=%s" % variant)
    res = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=variant)
    assert res[2][0] == gpu.GRID_TIMEOUT, res[2]
    monkeypatch.delenv("GLASS_AMD_GRID_SPIN_LIMIT")
    res = grid_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, single=variant)
    assert res[2][0] == gpu.CONVERGED
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, res, np.float64)


def grid_ws(glass, inp, ss, kp, max_iters, rel_tol, abs_tol, ws, keep, single, exclusive=True):
    t = {k: to_dev(v) for k, v in inp.items()}
    x = t["x0"].clone()
    iters = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros(2, dtype=x.dtype, device="cuda")
    glass.pcg_grid(x, t["S"], t["Pinv"], t["b"], ss, kp, max_iters, rel_tol, abs_tol,
                   iters, ws, status, rho, exclusive=exclusive, single_reduction=single,
                   keep_workspace=keep)
    torch.cuda.synchronize()
    return (x.cpu().numpy(), iters.cpu().numpy(), status.cpu().numpy(),
            rho.cpu().numpy().reshape(1, 2))


def test_grid_keep_workspace_sequence(gpu, monkeypatch, variant):
    """GLASS_GRID_KEEP_WORKSPACE: one workspace serves, in turn, the fp64
    chain, a solve that stops after its first barrier (rho_init = 0), the
    chain again, a smaller fp32 chain on another grid size, a forced timeout
    and a normal solve after it.  No clearing kernel runs after the first
    solve, so every stale word left there must fail its tag check: each
    result equals the same solve with the per-solve clearing (bit for bit),
    and the chain meets the oracle."""
    w = workloads.WORKLOADS[4]
    chain = workloads.generate(w)
    zero = dict(chain, b=np.zeros_like(chain["b"]))
    rng = np.random.default_rng(909)
    S, D = workloads.random_spd_strips(rng, 1, 6, 300, 0.1, np.float32)
    small = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, np.float32),
             "b": rng.standard_normal((1, 1800)).astype(np.float32),
             "x0": np.zeros((1, 1800), np.float32)}
    nbytes = max(gpu.pcg_grid_workspace_bytes(w.ss, w.kp, torch.float64),
                 gpu.pcg_grid_workspace_bytes(6, 300, torch.float32))
    kept = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fresh = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    seq = [("chain", chain, w.ss, w.kp, w.max_iters, w.rel_tol, None),
           ("rho_init = 0", zero, w.ss, w.kp, w.max_iters, w.rel_tol, None),
           ("chain again", chain, w.ss, w.kp, w.max_iters, w.rel_tol, None),
           ("small fp32 chain", small, 6, 300, 500, 1e-7, None),
           ("forced timeout", chain, w.ss, w.kp, w.max_iters, w.rel_tol, "0"),
           ("chain after the timeout", chain, w.ss, w.kp, w.max_iters, w.rel_tol, None),
           ("small fp32 chain again", small, 6, 300, 500, 1e-7, None)]
    for name, inp, ss, kp, mi, rel, spin in seq:
        say("grid kept workspace: %s single=%s" % (name, variant))
        if spin is not None:
            monkeypatch.setenv("GLASS_AMD_GRID_SPIN_LIMIT", spin)
        got = grid_ws(gpu, inp, ss, kp, mi, rel, 0.0, kept, True, variant)
        if spin is not None:
            assert got[2][0] == gpu.GRID_TIMEOUT, got[2]
            monkeypatch.delenv("GLASS_AMD_GRID_SPIN_LIMIT")
            continue
        ref = grid_ws(gpu, inp, ss, kp, mi, rel, 0.0, fresh, False, variant)
        for u, v in zip(ref, got):
            np.testing.assert_array_equal(u, v)
        assert got[2][0] == gpu.CONVERGED
        if name == "rho_init = 0":
            assert got[1][0] == 0
    res = grid_ws(gpu, chain, w.ss, w.kp, w.max_iters, w.rel_tol, 0.0, kept, True, variant)
    assert_pcg_parity(chain, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, res, np.float64)
