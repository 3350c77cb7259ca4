"""glass_pcg_grid_noalloc, the grid solve that allocates nothing (its exchange
area is the library's static per-device scratch), against glass_pcg_grid_ex
with a caller-owned workspace through the C ABI: the same kernels, so the same
bits, on two calls in a row, the second on a smaller problem (so the scratch
holds the first call's words when the second starts), in both forms and both
launches, and each result to the oracle bars of gpu_common."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads
from gpu_common import assert_pcg_parity, say, to_dev

pytestmark = pytest.mark.gpu


def run(glass, inp, ss, kp, max_iters, rel, noalloc, exclusive, single):
    t = {k: to_dev(v) for k, v in inp.items()}
    x = t["x0"].clone()
    iters = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros(2, dtype=x.dtype, device="cuda")
    if noalloc:
        glass.pcg_grid_noalloc(x, t["S"], t["Pinv"], t["b"], ss, kp, max_iters, rel, 0.0,
                               iters, status, rho, exclusive=exclusive, single_reduction=single)
    else:
        ws = torch.empty(glass.pcg_grid_workspace_bytes(ss, kp, x.dtype), dtype=torch.uint8,
                         device="cuda")
        glass.pcg_grid(x, t["S"], t["Pinv"], t["b"], ss, kp, max_iters, rel, 0.0, iters, ws,
                       status, rho, exclusive=exclusive, single_reduction=single)
    torch.cuda.synchronize()
    return (x.cpu().numpy(), iters.cpu().numpy(), status.cpu().numpy(),
            rho.cpu().numpy().reshape(1, 2))


def cases():
    """The kp=8192 ss=12 fp64 chain (block-tridiagonal Pinv), then a smaller
    fp32 chain (ss=6, kp=300, block-Jacobi Pinv)."""
    w = replace(workloads.WORKLOADS[4], pinv="tridiagonal")
    big = (workloads.generate(w), w.ss, w.kp, w.max_iters, w.rel_tol, np.float64)
    rng = np.random.default_rng(606)
    S, D = workloads.random_spd_strips(rng, 1, 6, 300, 0.1, np.float32)
    small = ({"S": S, "Pinv": workloads.block_jacobi_pinv(D, np.float32),
              "b": rng.standard_normal((1, 1800)).astype(np.float32),
              "x0": np.zeros((1, 1800), np.float32)}, 6, 300, 500, 1e-7, np.float32)
    return big, small


@pytest.mark.parametrize("exclusive", [False, True])
@pytest.mark.parametrize("single", [False, True])
def test_grid_noalloc_matches_workspace_call(gpu, exclusive, single):
    for inp, ss, kp, mi, rel, dt in cases():
        say("grid no-alloc ss=%d kp=%d %s exclusive=%s single=%s"
            % (ss, kp, np.dtype(dt).name, exclusive, single))
        got = run(gpu, inp, ss, kp, mi, rel, True, exclusive, single)
        ref = run(gpu, inp, ss, kp, mi, rel, False, exclusive, single)
        assert got[2][0] == gpu.CONVERGED
        for u, v in zip(ref, got):
            np.testing.assert_array_equal(u, v)
        assert_pcg_parity(inp, ss, kp, mi, rel, 0.0, got, dt)


def test_grid_noalloc_rejects_what_does_not_fit(gpu):
    """A grid whose exchange area exceeds the static scratch is refused with
    GLASS_EUNSUPPORTED before anything is launched (ss=64 fp64 on a chain
    long enough to need 1024 workgroups)."""
    ss, kp = 64, 4096
    n = ss * kp
    x = torch.zeros(n, dtype=torch.float64, device="cuda")
    S = torch.zeros(kp * ss * 3 * ss, dtype=torch.float64, device="cuda")
    it = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(gpu.GlassError) as ei:
        gpu.pcg_grid_noalloc(x, S, S, x, ss, kp, 10, 1e-10, 0.0, it)
    assert ei.value.code == -2
    assert "static scratch" in str(ei.value)
