"""Helpers for the GPU parity tests: run the HIP path through the C ABI on the
seeded inputs and compare with the CPU oracle at the stated tolerances.

Tolerances (stated here once, used by every GPU test):
* bdmv: |y_gpu - y_ref| <= 1e-5 * sum_c |S[br][i][c] * v[br*ss+c]| per row,
  with y_ref summed in float64 by the oracle.
* PCG: iteration count within +-2 of the oracle run in the same precision
  (the stopping decision is taken in the kernel's precision on both sides);
  x within relative L2 1e-4 (float32) / 1e-10 (float64) of the float64 oracle
  run for exactly the GPU's iteration count; the returned last r^T z meets
  the stopping criterion whenever the status says converged.
* PCG stopping point, independent of the kernel's own scalars: from the
  returned x, r = b - S x and z = Pinv r are recomputed in float64 by the
  oracle's matvec, and for every converged problem that took k >= 1
  iterations |r^T z| < CRIT_SLACK * thresh, with thresh = abs_tol + rel_tol *
  |rho_init| from the float64 oracle; and the float64 oracle stopped after
  k - 1 iterations has |r^T z| >= thresh / CRIT_SLACK (the kernel did not
  run on past the point where the criterion was first met by a wide margin).
  CRIT_SLACK covers the difference between the kernel's recurrence residual
  (rounded in its precision) and the true one, and the +-2 iteration slack:
  4 for float32, 2 for float64.
"""

import sys

import numpy as np
import torch

import oracle

BDMV_REL = 1e-5
X_REL = {np.float32: 1e-4, np.float64: 1e-10}
CRIT_SLACK = {np.float32: 4.0, np.float64: 2.0}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bdmv_gpu(glass, S, v, ss, kp, sentinel=float("nan")):
    St, vt = to_dev(S), to_dev(v)
    y = torch.full_like(vt, sentinel)
    glass.bdmv_batched(y, St, vt, ss, kp)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_bdmv_close(y_gpu, S, v, ss, kp, nthreads=8):
    B = y_gpu.shape[0]
    y_ref = oracle.bdmv(S, v, ss, kp, "f64", nthreads=nthreads)
    scale = oracle.bdmv(np.abs(np.asarray(S, np.float64)), np.abs(np.asarray(v, np.float64)),
                        ss, kp, "f64", nthreads=nthreads)
    yi = y_gpu.reshape(B, -1)[:, ss:-ss].astype(np.float64)
    err = np.abs(yi - y_ref[:, ss:-ss])
    bound = BDMV_REL * scale[:, ss:-ss]
    bad = err > bound
    assert not bad.any(), "bdmv parity: %d rows over 1e-5*row-abs-sum, worst %g" % (
        bad.sum(), float((err / np.maximum(scale[:, ss:-ss], 1e-300)).max()))


def pack_diagonal_blocks(P, ss, kp):
    """The D blocks of [L|D|R] Pinv strips, packed as [B, kp, ss, ss] (the
    GLASS_PCG_PINV_DIAGONAL_BLOCKS layout); a copy, no arithmetic."""
    B = P.shape[0]
    return np.ascontiguousarray(P.reshape(B, kp, ss, 3 * ss)[:, :, :, ss:2 * ss])


def pcg_gpu(glass, inp, ss, kp, max_iters, rel_tol, abs_tol, x0=None, pinv_block_diagonal=False,
            pinv_diagonal_blocks=False):
    t = {k: to_dev(v) for k, v in inp.items() if k in ("S", "b")}
    P = pack_diagonal_blocks(inp["Pinv"], ss, kp) if pinv_diagonal_blocks else inp["Pinv"]
    t["Pinv"] = to_dev(P)
    B = inp["b"].shape[0]
    x = to_dev(inp["x0"] if x0 is None else x0).clone()
    iters = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, 2), dtype=x.dtype, device="cuda")
    glass.pcg_batched(x, t["S"], t["Pinv"], t["b"], ss, kp, max_iters, rel_tol,
                      abs_tol, iters, status, rho, pinv_block_diagonal=pinv_block_diagonal,
                      pinv_diagonal_blocks=pinv_diagonal_blocks)
    torch.cuda.synchronize()
    return x.cpu().numpy(), iters.cpu().numpy(), status.cpu().numpy(), rho.cpu().numpy()


def true_rz(S, P, b, x, ss, kp, nthreads=8):
    """r^T z per problem with r = b - S x and z = Pinv r, all in float64 by
    the oracle's matvec (padded vectors with zero pads)."""
    B = b.shape[0]
    n = kp * ss
    xp = np.zeros((B, (kp + 2) * ss))
    xp[:, ss:ss + n] = np.asarray(x, np.float64).reshape(B, n)
    sx = oracle.bdmv(S, xp, ss, kp, "f64", nthreads=nthreads)[:, ss:ss + n]
    r = np.asarray(b, np.float64).reshape(B, n) - sx
    rp = np.zeros_like(xp)
    rp[:, ss:ss + n] = r
    z = oracle.bdmv(P, rp, ss, kp, "f64", nthreads=nthreads)[:, ss:ss + n]
    return np.einsum("ij,ij->i", r, z)


def assert_pcg_parity(inp, ss, kp, max_iters, rel_tol, abs_tol, result, dtype,
                      nthreads=8, x0=None):
    """x / iters / status / rho from the GPU against the oracle."""
    xg, itg, stg, rhog = result
    x0 = inp["x0"] if x0 is None else x0
    prec = "f32" if dtype == np.float32 else "f64"
    xo, ito, sto, rhoo = oracle.pcg(x0, inp["S"], inp["Pinv"], inp["b"], ss, kp,
                                    max_iters, rel_tol, abs_tol, prec, nthreads)
    assert np.all(np.abs(itg - ito) <= 2), "iteration counts differ by more than 2"
    conv = stg == oracle.CONVERGED
    assert np.array_equal(conv, sto == oracle.CONVERGED), "convergence status differs"
    # rho_init agrees with the oracle's
    np.testing.assert_allclose(rhog[:, 0], rhoo[:, 0], rtol=1e-4 if prec == "f32" else 1e-10)
    # the stopping criterion holds for every converged problem
    thresh = (np.asarray(abs_tol, dtype) + np.asarray(rel_tol, dtype) * np.abs(rhog[:, 0]).astype(dtype))
    assert np.all(np.abs(rhog[conv, 1]) < thresh[conv]), "final criterion not met"
    # x against the float64 oracle run for exactly the GPU's iteration count
    tol = X_REL[dtype]
    for k in np.unique(itg):
        sel = np.nonzero(itg == k)[0]
        xr, itr, _, _ = oracle.pcg(x0[sel], inp["S"][sel], inp["Pinv"][sel], inp["b"][sel],
                                   ss, kp, int(k), 0.0, 0.0, "f64", nthreads)
        num = np.linalg.norm(xg[sel].astype(np.float64) - xr, axis=1)
        den = np.maximum(np.linalg.norm(xr, axis=1), 1e-300)
        worst = float((num / den).max())
        assert worst <= tol, "x relative L2 error %g > %g at %d iterations" % (worst, tol, k)
    # the stopping point, from the returned x (see the module docstring)
    slack = CRIT_SLACK[dtype]
    rho_init64 = np.abs(true_rz(inp["S"], inp["Pinv"], inp["b"], x0, ss, kp, nthreads))
    thresh64 = abs_tol + rel_tol * rho_init64
    chk = np.nonzero(conv & (itg >= 1))[0]
    if chk.size:
        rz = np.abs(true_rz(inp["S"][chk], inp["Pinv"][chk], inp["b"][chk], xg[chk], ss, kp,
                            nthreads))
        ratio = rz / thresh64[chk]
        assert np.all(ratio < slack), \
            "true |r^T z| over %g x the criterion: worst ratio %g" % (slack, float(ratio.max()))
        worst_before = np.inf
        for k in np.unique(itg[chk]):
            sel = chk[itg[chk] == k]
            xm, _, _, _ = oracle.pcg(x0[sel], inp["S"][sel], inp["Pinv"][sel], inp["b"][sel],
                                     ss, kp, int(k) - 1, 0.0, 0.0, "f64", nthreads)
            rzm = np.abs(true_rz(inp["S"][sel], inp["Pinv"][sel], inp["b"][sel], xm, ss, kp,
                                 nthreads))
            before = rzm / thresh64[sel]
            worst_before = min(worst_before, float(before.min()))
            assert np.all(before >= 1.0 / slack), \
                "criterion already met %g x over at one iteration fewer than the GPU's %d" % (
                    float(before.min()), k)
        say("  stopping point: true |r^T z| / thresh <= %.3g at the GPU's x, >= %.3g one "
            "iteration earlier" % (float(ratio.max()), worst_before))
    return itg
