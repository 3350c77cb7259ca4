"""Properties of the seeded synthetic inputs (no method arithmetic here)."""

import numpy as np
import pytest

import oracle
import workloads


def test_generator_is_deterministic_and_prefix_stable():
    w = workloads.WORKLOADS[0]
    a = workloads.generate(w, n_problems=10)
    b = workloads.generate(w, n_problems=10)
    c = workloads.generate(w, n_problems=3, chunk=2)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
        np.testing.assert_array_equal(a[k][:3], c[k])


@pytest.mark.parametrize("cfg", [0, 2, 3])
def test_generated_matrix_is_symmetric_spd_with_margin(cfg):
    w = workloads.WORKLOADS[cfg]
    inp = workloads.generate(w, n_problems=2)
    for q in range(2):
        A = oracle.dense_expand(inp["S"][q].astype(np.float64), w.ss, w.kp)
        np.testing.assert_array_equal(A, A.T)
        lam = np.linalg.eigvalsh(A)
        # Gershgorin: lambda_min >= margin (up to the float32 rounding of S)
        assert lam[0] >= w.margin * (1 - 1e-3)
        # strict diagonal dominance over the full row
        d = np.diag(A)
        off = np.abs(A).sum(1) - np.abs(d)
        np.testing.assert_allclose(d - off, w.margin, rtol=0, atol=1e-4)


def test_off_matrix_blocks_and_pads_are_zero():
    w = workloads.WORKLOADS[1]
    inp = workloads.generate(w, n_problems=3)
    S, v = inp["S"], inp["v"]
    assert S.shape == (3, w.kp, w.ss, 3 * w.ss) and S.dtype == np.float32
    assert np.all(S[:, 0, :, :w.ss] == 0) and np.all(S[:, -1, :, 2 * w.ss:] == 0)
    assert np.all(v[:, :w.ss] == 0) and np.all(v[:, -w.ss:] == 0)
    assert v.shape == (3, (w.kp + 2) * w.ss)


def test_pinv_is_block_jacobi_inverse():
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w, n_problems=2)
    S = inp["S"].astype(np.float64)
    P = inp["Pinv"].astype(np.float64)
    ss = w.ss
    assert np.all(P[..., :ss] == 0) and np.all(P[..., 2 * ss:] == 0)
    prod = np.einsum("bkij,bkjl->bkil", P[..., ss:2 * ss], S[..., ss:2 * ss])
    np.testing.assert_allclose(prod, np.broadcast_to(np.eye(ss), prod.shape), atol=1e-5)


def test_config_table_matches_stated_workloads():
    c = workloads.WORKLOADS
    assert (c[0].ss, c[0].kp, c[0].n_problems, c[0].dtype) == (6, 32, 64, np.float32)
    assert (c[1].ss, c[1].kp, c[1].n_problems, c[1].kind) == (14, 64, 8192, "bdmv")
    assert (c[2].ss, c[2].kp, c[2].n_problems, c[2].margin) == (14, 32, 4096, 0.2)
    assert (c[3].ss, c[3].kp, c[3].n_problems, c[3].max_iters) == (21, 64, 2048, 500)
    assert (c[4].ss, c[4].kp, c[4].dtype, c[4].rel_tol) == (12, 8192, np.float64, 1e-10)


@pytest.mark.parametrize("ss,kp,margin", [(2, 5, 0.3), (6, 8, 0.1), (14, 4, 0.2), (3, 1, 0.5)])
def test_tridiagonal_pinv_is_the_dense_first_order_inverse_and_spd(ss, kp, margin):
    """pinv="tridiagonal": built from its definition with dense matrices
    (Pinv = D^-1 - D^-1 E D^-1, D the block diagonal of the expanded S, E the
    rest), symmetric, positive definite, non-zero L/R blocks for kp > 1, zero
    off-matrix blocks, and a better preconditioner than block Jacobi
    (condition number of Pinv S no larger)."""
    rng = np.random.default_rng(ss * 31 + kp)
    S, D = workloads.random_spd_strips(rng, 2, ss, kp, margin)
    P = workloads.block_tridiagonal_pinv(S, D)
    Pj = workloads.block_jacobi_pinv(D)
    assert np.all(P[:, 0, :, :ss] == 0) and np.all(P[:, -1, :, 2 * ss:] == 0)
    if kp > 1:
        assert np.abs(P[:, 1:, :, :ss]).min(axis=(2, 3)).max() > 0
        assert np.all(np.abs(P[:, :-1, :, 2 * ss:]).sum(axis=(2, 3)) > 0)
    n = kp * ss
    for q in range(2):
        A = oracle.dense_expand(S[q], ss, kp)
        Dd = np.zeros_like(A)
        for br in range(kp):
            sl = slice(br * ss, (br + 1) * ss)
            Dd[sl, sl] = A[sl, sl]
        E = A - Dd
        Di = np.linalg.inv(Dd)
        M = oracle.dense_expand(P[q], ss, kp)
        np.testing.assert_allclose(M, Di - Di @ E @ Di, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(M, M.T, rtol=0, atol=1e-15)
        lam = np.linalg.eigvalsh(M)
        assert lam[0] > 0, lam[0]
        # Pinv S is similar to I - F^2 with F = D^-1/2 E D^-1/2: eigenvalues in (0, 1]
        ev = np.sort(np.linalg.eigvals(M @ A).real)
        assert ev[0] > 0 and ev[-1] <= 1 + 1e-12
        evj = np.sort(np.linalg.eigvals(oracle.dense_expand(Pj[q], ss, kp) @ A).real)
        assert ev[-1] / ev[0] <= evj[-1] / evj[0] * (1 + 1e-9)
        assert M.shape == (n, n)


def test_generate_tridiagonal_pinv_option():
    """The option changes only Pinv: S, b and x0 are the same draws, Pinv's D
    blocks are the block-Jacobi inverse and its L/R blocks are not zero."""
    from dataclasses import replace
    w = workloads.WORKLOADS[2]
    a = workloads.generate(w, n_problems=3)
    b = workloads.generate(replace(w, pinv="tridiagonal"), n_problems=3)
    for k in ("S", "b", "x0"):
        np.testing.assert_array_equal(a[k], b[k])
    ss = w.ss
    np.testing.assert_array_equal(a["Pinv"][..., ss:2 * ss], b["Pinv"][..., ss:2 * ss])
    assert np.count_nonzero(b["Pinv"][:, :, :, 2 * ss:]) > 0
    assert np.count_nonzero(b["Pinv"][:, 1:, :, :ss]) > 0
    with pytest.raises(ValueError):
        workloads.generate(replace(w, pinv="nonsense"), n_problems=1)
