"""The several-problems-per-wave placement (16 or 32 lanes per problem, no
workgroup barriers) against the workgroup placement and the oracle through
the C ABI.  Its dots rebuild the workgroup's chunk-ordered sums from the same
DPP steps, so every output is bit-identical to the default placement; each
run also meets the oracle bars of gpu_common."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import assert_pcg_parity, pcg_gpu, say

pytestmark = pytest.mark.gpu


def both(gpu, monkeypatch, inp, ss, kp, max_iters, rel, abs_tol, **kw):
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "0")
    ref = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol, **kw)
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "1")
    got = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol, **kw)
    monkeypatch.delenv("GLASS_AMD_PCG_MULTI")
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    return got


@pytest.mark.parametrize("B,pinv", [(64, "block_jacobi"), (64, "tridiagonal"),
                                    (4096, "block_jacobi"), (37, "tridiagonal")])
def test_multi_small_workload(gpu, monkeypatch, B, pinv):
    """The ss=6 kp=32 workload (192 rows: 32 lanes x 6 rows, two problems
    per wave) at its 64 problems, at 4096, and at 37 (a partly filled wave
    and workgroup)."""
    w = replace(workloads.WORKLOADS[0], pinv=pinv)
    inp = workloads.generate(w, n_problems=B)
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "1")
    assert gpu.pcg_batched_placement(w.ss, w.kp, torch.float32) == \
        gpu.PLACEMENT_SEVERAL_PER_WAVE
    assert gpu.pcg_batched_pinned_rows(w.ss, w.kp, torch.float32) == 0
    say("pcg cfg0 B=%d Pinv=%s several problems per wave" % (B, pinv))
    got = both(gpu, monkeypatch, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    assert np.all(got[2] == gpu.CONVERGED)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)


@pytest.mark.parametrize("kp,B,dtype", [
    (1, 5, np.float32), (2, 9, np.float32), (5, 13, np.float32),    # 16 lanes, 1-2 rows
    (11, 6, np.float32), (16, 17, np.float32),                      # 16 lanes, 5 and 6 rows
    (20, 7, np.float32), (27, 3, np.float32),                       # 32 lanes, 4 and 6 rows
    (3, 11, np.float64), (8, 5, np.float64), (12, 4, np.float64),   # float64: 16 lanes
    (16, 3, np.float64),                                            # float64: 32 lanes, 3 rows
])
def test_multi_shapes(gpu, monkeypatch, kp, B, dtype):
    ss = 6
    rng = np.random.default_rng(kp * 31 + B)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2)
    P = workloads.block_tridiagonal_pinv(S, D, dtype) if kp % 2 else \
        workloads.block_jacobi_pinv(D, dtype)
    inp = {"S": S.astype(dtype), "Pinv": P, "b": rng.standard_normal((B, kp * ss)).astype(dtype),
           "x0": rng.standard_normal((B, kp * ss)).astype(dtype)}
    rel = 1e-8 if dtype == np.float32 else 1e-14
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "1")
    assert gpu.pcg_batched_placement(ss, kp, tdt) == gpu.PLACEMENT_SEVERAL_PER_WAVE
    say("pcg several per wave ss=6 kp=%d B=%d %s" % (kp, B, np.dtype(dtype).name))
    got = both(gpu, monkeypatch, inp, ss, kp, 300, rel, 0.0)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, got, dtype)


def test_multi_status_cases_in_one_wave(gpu, monkeypatch):
    """Breakdown (negative definite, NaN), rho_init = 0, max_iters = 0 and an
    exhausted max_iters among problems that share waves: statuses match the
    oracle and every output matches the workgroup placement bit for bit."""
    ss, kp, B = 6, 32, 6
    rng = np.random.default_rng(66)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2, np.float32)
    P = workloads.block_jacobi_pinv(D, np.float32)
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    x0 = rng.standard_normal((B, kp * ss)).astype(np.float32)
    S[1] = -S[1]
    b[2] = 0.0
    x0[2] = 0.0
    b[3, 7] = np.nan
    inp = {"S": S, "Pinv": P, "b": b, "x0": x0}
    for max_iters, rel, abs_tol in ((60, 1e-6, 0.0), (0, 1e-6, 0.0), (2, 0.0, 0.0),
                                    (60, 0.0, 1e30)):
        say("pcg several per wave status cases max_iters=%d abs_tol=%g" % (max_iters, abs_tol))
        x, it, st, _ = both(gpu, monkeypatch, inp, ss, kp, max_iters, rel, abs_tol)
        if max_iters == 60 and abs_tol == 0.0:
            _, ito, sto, _ = oracle.pcg(x0, S, P, b, ss, kp, 60, 1e-6, 0.0, "f32")
            np.testing.assert_array_equal(st, sto)
            assert st[1] == gpu.BREAKDOWN and st[3] == gpu.BREAKDOWN
            assert st[2] == gpu.CONVERGED and it[2] == 0 and np.all(x[2] == 0)
            assert np.all(np.abs(it - ito) <= 2)
        if max_iters == 0:
            assert np.all(it == 0) and st[0] == gpu.MAX_ITERS
        if max_iters == 2:
            assert np.all(it[[0, 4, 5]] == 2) and np.all(st[[0, 4, 5]] == gpu.MAX_ITERS)


def test_multi_default_choice(gpu, monkeypatch):
    """Left to itself the library takes this placement for chains of at most
    16 rows (where it was measured faster) and the workgroup placement
    otherwise; GLASS_AMD_PCG_MULTI=0 switches it off."""
    monkeypatch.delenv("GLASS_AMD_PCG_MULTI", raising=False)
    for kp in (1, 2):
        assert gpu.pcg_batched_placement(6, kp, torch.float32) == gpu.PLACEMENT_SEVERAL_PER_WAVE
        assert gpu.pcg_batched_placement(6, kp, torch.float64) == gpu.PLACEMENT_SEVERAL_PER_WAVE
    for kp in (3, 32):
        assert gpu.pcg_batched_placement(6, kp, torch.float32) == gpu.PLACEMENT_RESIDENT
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "0")
    assert gpu.pcg_batched_placement(6, 2, torch.float32) == gpu.PLACEMENT_RESIDENT


def test_multi_not_for_other_shapes(gpu, monkeypatch):
    """Shapes it does not cover keep their placement: other state sizes,
    more than 192 rows, packed D blocks."""
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "1")
    assert gpu.pcg_batched_placement(14, 32, torch.float32) == gpu.PLACEMENT_RESIDENT
    assert gpu.pcg_batched_placement(6, 33, torch.float32) != gpu.PLACEMENT_SEVERAL_PER_WAVE
    assert gpu.pcg_batched_placement(6, 32, torch.float32, pinv_diagonal_blocks=True) != \
        gpu.PLACEMENT_SEVERAL_PER_WAVE
    assert gpu.pcg_batched_placement(6, 17, torch.float64) != gpu.PLACEMENT_SEVERAL_PER_WAVE
