"""Resident rows with the Pinv rows brought in through each wave's LDS stage
by direct loads, and the S rows either straight into registers or through
the same stage first (GLASS_AMD_PCG_RESD_S_STAGE; by default for rows of
128 bytes or more): the same values in the same registers and the same
steps in the same order as the plain resident load
(GLASS_AMD_PCG_RES_DMA=0), so bit-identical outputs, and the oracle bars of
gpu_common."""

from dataclasses import replace

import numpy as np
import pytest

import oracle
import workloads
from gpu_common import assert_pcg_parity, pcg_gpu, say

pytestmark = pytest.mark.gpu


def both(gpu, monkeypatch, inp, ss, kp, max_iters, rel, abs_tol):
    monkeypatch.setenv("GLASS_AMD_PCG_RES_DMA", "0")
    ref = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
    monkeypatch.delenv("GLASS_AMD_PCG_RES_DMA")
    got = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    for s_stage in ("0", "1"):
        monkeypatch.setenv("GLASS_AMD_PCG_RESD_S_STAGE", s_stage)
        alt = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
        for u, v in zip(ref, alt):
            np.testing.assert_array_equal(u, v)
    monkeypatch.delenv("GLASS_AMD_PCG_RESD_S_STAGE")
    return got


@pytest.mark.parametrize("cfg,pinv", [(2, "block_jacobi"), (2, "tridiagonal"),
                                      (0, "block_jacobi"), (0, "tridiagonal")])
def test_resident_dma_workloads(gpu, monkeypatch, cfg, pinv):
    """The ss=14 kp=32 workload (4096 problems) and the ss=6 kp=32 workload
    (64 problems), both preconditioners."""
    w = replace(workloads.WORKLOADS[cfg], pinv=pinv)
    inp = workloads.generate(w)
    say("pcg cfg%d Pinv=%s: Pinv rows through the LDS stage vs straight loads" % (cfg, pinv))
    got = both(gpu, monkeypatch, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    assert np.all(got[2] == gpu.CONVERGED)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)


@pytest.mark.parametrize("ss,kp,B,dtype", [
    (14, 20, 77, np.float32),     # 280 rows: ragged last chunk (masked tail loads)
    (12, 50, 9, np.float32),      # 600 rows, 10 waves
    (6, 32, 4096, np.float32),
    (6, 40, 30, np.float64),
    (14, 5, 20, np.float32),      # one wave, ragged
    (12, 1, 7, np.float32),       # one block-row
])
def test_resident_dma_shapes(gpu, monkeypatch, ss, kp, B, dtype):
    rng = np.random.default_rng(ss * 1000 + kp + B)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2)
    P = workloads.block_tridiagonal_pinv(S, D, dtype) if B % 2 else \
        workloads.block_jacobi_pinv(D, dtype)
    inp = {"S": S.astype(dtype), "Pinv": P, "b": rng.standard_normal((B, kp * ss)).astype(dtype),
           "x0": rng.standard_normal((B, kp * ss)).astype(dtype)}
    rel = 1e-7 if dtype == np.float32 else 1e-14
    say("pcg resident, Pinv through the stage: ss=%d kp=%d B=%d %s"
        % (ss, kp, B, np.dtype(dtype).name))
    got = both(gpu, monkeypatch, inp, ss, kp, 300, rel, 0.0)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, got, dtype)


def test_resident_dma_status_cases(gpu, monkeypatch):
    """Breakdown (negative definite, NaN), rho_init = 0, max_iters = 0 and
    exhausted: every output equals the plain resident load."""
    ss, kp, B = 14, 32, 300
    rng = np.random.default_rng(14)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2, np.float32)
    P = workloads.block_jacobi_pinv(D, np.float32)
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    x0 = rng.standard_normal((B, kp * ss)).astype(np.float32)
    S[1::37] = -S[1::37]
    b[2::41] = 0.0
    x0[2::41] = 0.0
    b[3::43, 5] = np.nan
    inp = {"S": S, "Pinv": P, "b": b, "x0": x0}
    for max_iters, rel, abs_tol in ((60, 1e-6, 0.0), (0, 1e-6, 0.0), (2, 0.0, 0.0),
                                    (60, 0.0, 1e30)):
        say("pcg resident via stage, status cases max_iters=%d abs_tol=%g" % (max_iters, abs_tol))
        x, it, st, _ = both(gpu, monkeypatch, inp, ss, kp, max_iters, rel, abs_tol)
        if max_iters == 60 and abs_tol == 0.0:
            _, ito, sto, _ = oracle.pcg(x0, S, P, b, ss, kp, 60, 1e-6, 0.0, "f32")
            np.testing.assert_array_equal(st, sto)
            assert np.all(st[1::37] == gpu.BREAKDOWN) and np.all(st[2::41] == gpu.CONVERGED)
            assert np.all(np.abs(it - ito) <= 2)
