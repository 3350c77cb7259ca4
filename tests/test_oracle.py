"""Pins of the CPU oracle against things other than itself.

Each test names the plausible oracle mistake it would catch.  Sources: the
GLASS user guide page "Block-tridiagonal Solves" (layout, padded vectors, the
PCG stopping rule) and textbook facts about conjugate gradients (finite
termination, orthogonality, monotone energy error, hand-derived iterates).
"""

import numpy as np
import pytest

import oracle
import workloads
from conftest import frac_array, read_golden


# ---------------------------------------------------------------------------
# bdmv
# ---------------------------------------------------------------------------

def test_bdmv_golden_hand_example():
    """Hand-derived integers: catches a wrong window offset, a wrong output
    offset, L/R swapped, or off-matrix blocks leaking into the result."""
    g = read_golden("bdmv_ss2_kp2.txt")
    ss, kp = int(g["ss"][0]), int(g["kp"][0])
    S = frac_array(g["S"]).reshape(1, -1)
    v = frac_array(g["v"]).reshape(1, -1)
    y = oracle.bdmv(S, v, ss, kp, precision="f64", y=np.full((1, 8), -99.0))
    np.testing.assert_array_equal(y[0, ss:-ss], frac_array(g["y_interior"]))
    # the pads of y are not written
    np.testing.assert_array_equal(y[0, :ss], [-99.0] * ss)
    np.testing.assert_array_equal(y[0, -ss:], [-99.0] * ss)
    y32 = oracle.bdmv(S.astype(np.float32), v.astype(np.float32), ss, kp, "f32")
    np.testing.assert_array_equal(y32[0, ss:-ss], frac_array(g["y_interior"]))


def _random_blocks(rng, ss, kp):
    L = rng.standard_normal((kp, ss, ss))
    D = rng.standard_normal((kp, ss, ss))
    R = rng.standard_normal((kp, ss, ss))
    return L, D, R


def _strips_from_blocks(L, D, R):
    return np.concatenate([L, D, R], axis=-1)  # [kp, ss, 3ss]


def _dense_from_blocks(L, D, R):
    """The block-tridiagonal matrix written out from its definition: block
    (br, br-1) = L_br, (br, br) = D_br, (br, br+1) = R_br."""
    kp, ss, _ = D.shape
    n = kp * ss
    A = np.zeros((n, n))
    for br in range(kp):
        A[br * ss:(br + 1) * ss, br * ss:(br + 1) * ss] = D[br]
        if br > 0:
            A[br * ss:(br + 1) * ss, (br - 1) * ss:br * ss] = L[br]
        if br < kp - 1:
            A[br * ss:(br + 1) * ss, (br + 1) * ss:(br + 2) * ss] = R[br]
    return A


@pytest.mark.parametrize("ss,kp", [(1, 1), (1, 5), (2, 3), (3, 1), (5, 7), (14, 4)])
def test_bdmv_matches_dense_product(ss, kp):
    """Random non-symmetric blocks: catches transposed blocks, a block placed
    in the wrong column, and an off-by-one in the window."""
    rng = np.random.default_rng(ss * 100 + kp)
    L, D, R = _random_blocks(rng, ss, kp)
    A = _dense_from_blocks(L, D, R)
    x = rng.standard_normal(kp * ss)
    v = np.zeros((kp + 2) * ss)
    v[ss:-ss] = x
    y = oracle.bdmv(_strips_from_blocks(L, D, R)[None], v[None], ss, kp)
    np.testing.assert_allclose(y[0, ss:-ss], A @ x, rtol=1e-13, atol=1e-13)
    # the oracle's own dense expansion agrees exactly with the definition
    np.testing.assert_array_equal(
        oracle.dense_expand(_strips_from_blocks(L, D, R), ss, kp), A)


def test_bdmv_zero_pad_invariance():
    """Finite garbage in L_0 and R_{kp-1} must not change y (they multiply
    the zero pads)."""
    rng = np.random.default_rng(7)
    ss, kp, B = 4, 6, 3
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 1.0)
    v = np.zeros((B, (kp + 2) * ss))
    v[:, ss:-ss] = rng.standard_normal((B, kp * ss))
    y0 = oracle.bdmv(S, v, ss, kp)
    S2 = S.copy()
    S2[:, 0, :, :ss] = rng.uniform(-1e3, 1e3, (B, ss, ss))
    S2[:, -1, :, 2 * ss:] = rng.uniform(-1e3, 1e3, (B, ss, ss))
    np.testing.assert_array_equal(oracle.bdmv(S2, v, ss, kp), y0)


def test_bdmv_identity_strips():
    ss, kp, B = 3, 5, 2
    S = workloads.identity_pinv(B, ss, kp)
    rng = np.random.default_rng(3)
    v = np.zeros((B, (kp + 2) * ss))
    v[:, ss:-ss] = rng.standard_normal((B, kp * ss))
    y = oracle.bdmv(S, v, ss, kp)
    np.testing.assert_array_equal(y[:, ss:-ss], v[:, ss:-ss])


def test_bdmv_symmetry_of_generated_matrix():
    """u^T (S v) = v^T (S u) for the generator's symmetric S: catches an
    oracle that reads L as R^T instead of L itself (or vice versa)."""
    rng = np.random.default_rng(11)
    ss, kp = 5, 9
    S, _ = workloads.random_spd_strips(rng, 1, ss, kp, 0.5)
    u = np.zeros((1, (kp + 2) * ss))
    v = np.zeros_like(u)
    u[:, ss:-ss] = rng.standard_normal(kp * ss)
    v[:, ss:-ss] = rng.standard_normal(kp * ss)
    Su = oracle.bdmv(S, u, ss, kp)
    Sv = oracle.bdmv(S, v, ss, kp)
    a = float(u[0, ss:-ss] @ Sv[0, ss:-ss])
    b = float(v[0, ss:-ss] @ Su[0, ss:-ss])
    assert abs(a - b) <= 1e-12 * max(1.0, abs(a))


def test_bdmv_f32_within_dot_error_bound():
    """Float32 accumulation stays inside the classical dot-product bound
    gamma_k * sum|a_i b_i| (Higham, Accuracy and Stability, sec. 3.1)."""
    w = workloads.WORKLOADS[1]
    inp = workloads.generate(w, n_problems=4)
    S, v = inp["S"], inp["v"]
    y64 = oracle.bdmv(S, v, w.ss, w.kp, "f64")
    y32 = oracle.bdmv(S, v, w.ss, w.kp, "f32")
    absS = np.abs(S.astype(np.float64))
    absv = np.abs(v.astype(np.float64))
    scale = oracle.bdmv(absS, absv, w.ss, w.kp, "f64")
    k = 3 * w.ss
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    err = np.abs(y32.astype(np.float64) - y64)[:, w.ss:-w.ss]
    assert np.all(err <= gamma * scale[:, w.ss:-w.ss] + 1e-30)


def test_bdmv_threads_bitwise_equal():
    w = workloads.WORKLOADS[1]
    inp = workloads.generate(w, n_problems=9)
    a = oracle.bdmv(inp["S"], inp["v"], w.ss, w.kp, "f32", nthreads=1)
    b = oracle.bdmv(inp["S"], inp["v"], w.ss, w.kp, "f32", nthreads=4)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# dense Cholesky
# ---------------------------------------------------------------------------

def test_cholesky_solve_matches_lu():
    rng = np.random.default_rng(5)
    M = rng.standard_normal((9, 9))
    A = M @ M.T + 9 * np.eye(9)
    b = rng.standard_normal(9)
    np.testing.assert_allclose(oracle.cholesky_solve(A, b),
                               np.linalg.solve(A, b), rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.cholesky_solve(-A, b)


# ---------------------------------------------------------------------------
# pcg
# ---------------------------------------------------------------------------

def _cg2x2_problem(embedding, pinv_diag=None):
    """The 2x2 system A = [[4,1],[1,3]] as strips in either embedding."""
    if embedding == "ss1":
        ss, kp = 1, 2
        S = np.array([[[[9.0, 4.0, 1.0]], [[1.0, 3.0, 9.0]]]])  # L_0, R_1 garbage
        P = np.zeros_like(S)
        d = [1.0, 1.0] if pinv_diag is None else pinv_diag
        P[0, 0, 0, 1], P[0, 1, 0, 1] = d
    else:
        ss, kp = 2, 1
        S = np.zeros((1, 1, 2, 6))
        S[0, 0, :, 2:4] = [[4.0, 1.0], [1.0, 3.0]]
        S[0, 0, :, :2] = 5.0   # off-matrix garbage
        S[0, 0, :, 4:] = -5.0
        P = np.zeros_like(S)
        d = [1.0, 1.0] if pinv_diag is None else pinv_diag
        P[0, 0, 0, 2], P[0, 0, 1, 3] = d
    return S, P, ss, kp


@pytest.mark.parametrize("embedding", ["ss1", "ss2"])
def test_pcg_golden_textbook_cg(embedding):
    """Hand-derived CG iterates: catches a wrong sign in the residual update,
    alpha or beta inverted, or a wrong search-direction update."""
    g = read_golden("cg_2x2.txt")
    b = frac_array(g["b"])
    S, P, ss, kp = _cg2x2_problem(embedding)
    x0 = frac_array(g["identity.x0"])
    for k, key in ((1, "identity.x1"), (2, "identity.x2")):
        x, it, st, _ = oracle.pcg(x0[None], S, P, b[None], ss, kp, k, 0.0, 0.0)
        assert it[0] == k and st[0] == oracle.MAX_ITERS
        np.testing.assert_allclose(x[0], frac_array(g[key]), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("embedding", ["ss1", "ss2"])
def test_pcg_golden_jacobi_preconditioned(embedding):
    """Hand-derived preconditioned iterates: catches z = r (preconditioner
    ignored), rho = r^T r instead of r^T z, or Pinv applied to the wrong
    vector."""
    g = read_golden("cg_2x2.txt")
    b = frac_array(g["b"])
    S, P, ss, kp = _cg2x2_problem(embedding, frac_array(g["jacobi.pinv_diag"]))
    x0 = frac_array(g["jacobi.x0"])
    x1, it, _, _ = oracle.pcg(x0[None], S, P, b[None], ss, kp, 1, 0.0, 0.0)
    np.testing.assert_allclose(x1[0], frac_array(g["jacobi.x1"]), rtol=1e-14)
    r1 = b - np.array([[4.0, 1.0], [1.0, 3.0]]) @ x1[0]
    np.testing.assert_allclose(r1, frac_array(g["jacobi.r1"]), rtol=1e-13)
    x2, it, _, _ = oracle.pcg(x0[None], S, P, b[None], ss, kp, 2, 0.0, 0.0)
    np.testing.assert_allclose(x2[0], frac_array(g["jacobi.x2"]), rtol=1e-13)


def test_pcg_matches_dense_cholesky_tiny():
    """kp=4, ss=2 (n=8), fp64 with a tolerance far below rounding: the
    converged x equals a dense Cholesky solve and numpy's LU solve."""
    rng = np.random.default_rng(42)
    ss, kp, B = 2, 4, 6
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.3)
    P = workloads.block_jacobi_pinv(D)
    b = rng.standard_normal((B, kp * ss))
    x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 100, 1e-28, 0.0)
    for q in range(B):
        A = oracle.dense_expand(S[q], ss, kp)
        xs = oracle.cholesky_solve(A, b[q])
        np.testing.assert_allclose(x[q], xs, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(x[q], np.linalg.solve(A, b[q]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("ss,kp", [(1, 8), (2, 4), (4, 2), (3, 3)])
def test_pcg_identity_finite_termination(ss, kp):
    """CG with Pinv = I terminates in at most n steps in exact arithmetic;
    in fp64 on a well-conditioned n <= 9 system the relative residual
    criterion 1e-24 is met within n iterations."""
    rng = np.random.default_rng(ss * 10 + kp)
    S, _ = workloads.random_spd_strips(rng, 4, ss, kp, 0.5)
    P = workloads.identity_pinv(4, ss, kp)
    b = rng.standard_normal((4, kp * ss))
    x, it, st, rho = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 50, 1e-24, 0.0)
    assert np.all(st == oracle.CONVERGED)
    assert np.all(it <= kp * ss), it


def test_pcg_block_diagonal_exact_preconditioner_one_iteration():
    """Block-diagonal S with its exact block-Jacobi inverse: Pinv S = I, so
    PCG converges in exactly one iteration to x = S^-1 b."""
    rng = np.random.default_rng(9)
    ss, kp, B = 4, 5, 3
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.5, offdiag=False)
    P = workloads.block_jacobi_pinv(D)
    b = rng.standard_normal((B, kp * ss))
    x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 20, 1e-20, 0.0)
    assert np.all(it == 1) and np.all(st == oracle.CONVERGED)
    for q in range(B):
        A = oracle.dense_expand(S[q], ss, kp)
        np.testing.assert_allclose(x[q], np.linalg.solve(A, b[q]), rtol=1e-12)


def test_pcg_scaled_identity_one_iteration():
    ss, kp, B = 3, 4, 2
    S = 2.5 * workloads.identity_pinv(B, ss, kp)
    P = workloads.identity_pinv(B, ss, kp)
    b = np.random.default_rng(1).standard_normal((B, kp * ss))
    x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 10, 1e-20, 0.0)
    assert np.all(it == 1)
    np.testing.assert_allclose(x, b / 2.5, rtol=1e-15)


def test_pcg_identical_blocks_distinct_eigenvalues_bound():
    """Block-diagonal S with the same D block everywhere has at most ss
    distinct eigenvalues, so CG (Pinv = I) terminates in <= ss iterations."""
    rng = np.random.default_rng(21)
    ss, kp = 3, 6
    _, D = workloads.random_spd_strips(rng, 1, ss, 1, 0.5, offdiag=False)
    S = np.zeros((1, kp, ss, 3 * ss))
    S[0, :, :, ss:2 * ss] = D[0, 0]
    P = workloads.identity_pinv(1, ss, kp)
    b = rng.standard_normal((1, kp * ss))
    x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 50, 1e-26, 0.0)
    assert st[0] == oracle.CONVERGED and it[0] <= ss


def _residual_and_z(S, P, x, b, ss, kp):
    A = oracle.dense_expand(S, ss, kp)
    M = oracle.dense_expand(P, ss, kp)
    r = b - A @ x
    return A, r, M @ r


def test_pcg_orthogonality_and_monotone_energy_error():
    """Textbook PCG invariants on a kp=6, ss=3 problem with a full
    block-tridiagonal Pinv: r_k^T z_j = 0 for j < k (up to rounding) and the
    S-norm error ||x_k - x*||_S never increases."""
    rng = np.random.default_rng(77)
    ss, kp = 3, 6
    S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.4)
    # a symmetric positive definite block-tridiagonal preconditioner
    P, _ = workloads.random_spd_strips(rng, 1, ss, kp, 2.0)
    b = rng.standard_normal((1, kp * ss))
    A = oracle.dense_expand(S[0], ss, kp)
    xs = np.linalg.solve(A, b[0])
    xs_list, rs, zs = [], [], []
    for k in range(0, 8):
        x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, k, 0.0, 0.0)
        assert it[0] == k
        _, r, z = _residual_and_z(S[0], P[0], x[0], b[0], ss, kp)
        xs_list.append(x[0])
        rs.append(r)
        zs.append(z)
    for k in range(1, 8):
        for j in range(k):
            rel = abs(rs[k] @ zs[j]) / (np.linalg.norm(rs[k]) * np.linalg.norm(zs[j]) + 1e-300)
            assert rel < 1e-8, (k, j, rel)
    err = [float((xk - xs) @ A @ (xk - xs)) for xk in xs_list]
    for a, c in zip(err, err[1:]):
        assert c <= a * (1 + 1e-12) + 1e-28


def test_pcg_iteration_count_is_first_to_meet_criterion():
    """The returned x meets |r^T z| < abs + rel*|rho_init| (recomputed densely
    in fp64) and one iteration fewer does not: catches a test placed before
    or after the right point, and a non-strict comparison drift."""
    w = workloads.WORKLOADS[0]
    inp = workloads.generate(w, n_problems=8)
    S = inp["S"].astype(np.float64)
    P = inp["Pinv"].astype(np.float64)
    b = inp["b"].astype(np.float64)
    x, it, st, rho = oracle.pcg(np.zeros_like(b), S, P, b, w.ss, w.kp,
                                w.max_iters, w.rel_tol, w.abs_tol)
    assert np.all(st == oracle.CONVERGED) and np.all(it >= 2)
    for q in range(b.shape[0]):
        _, r0, z0 = _residual_and_z(S[q], P[q], np.zeros(w.n), b[q], w.ss, w.kp)
        rho_init = abs(r0 @ z0)
        np.testing.assert_allclose(rho[q, 0], r0 @ z0, rtol=1e-12)
        thresh = w.abs_tol + w.rel_tol * rho_init
        _, r, z = _residual_and_z(S[q], P[q], x[q], b[q], w.ss, w.kp)
        assert abs(r @ z) < thresh * 1.01
        assert abs(rho[q, 1]) < thresh
        xm, itm, stm, rhom = oracle.pcg(np.zeros((1, w.n)), S[q:q + 1], P[q:q + 1],
                                        b[q:q + 1], w.ss, w.kp, int(it[q]) - 1,
                                        w.rel_tol, w.abs_tol)
        assert stm[0] == oracle.MAX_ITERS and abs(rhom[0, 1]) >= thresh


def test_pcg_status_cases():
    rng = np.random.default_rng(4)
    ss, kp = 2, 3
    S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.5)
    P = workloads.block_jacobi_pinv(D)
    b = rng.standard_normal((1, kp * ss))
    x0 = rng.standard_normal((1, kp * ss))
    # b = 0 and x0 = 0: rho_init == 0 -> converged, nothing done
    x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, np.zeros_like(b), ss, kp, 10, 1e-6, 0.0)
    assert it[0] == 0 and st[0] == oracle.CONVERGED and np.all(x == 0)
    # huge abs_tol: converged before the loop, x0 returned unchanged
    x, it, st, _ = oracle.pcg(x0, S, P, b, ss, kp, 10, 0.0, 1e30)
    assert it[0] == 0 and st[0] == oracle.CONVERGED
    np.testing.assert_array_equal(x, x0)
    # max_iters = 0 and not converged
    x, it, st, _ = oracle.pcg(x0, S, P, b, ss, kp, 0, 1e-6, 0.0)
    assert it[0] == 0 and st[0] == oracle.MAX_ITERS
    np.testing.assert_array_equal(x, x0)
    # negative definite S: p^T S p < 0 at the first step -> breakdown
    x, it, st, _ = oracle.pcg(x0, -S, P, b, ss, kp, 10, 1e-6, 0.0)
    assert it[0] == 0 and st[0] == oracle.BREAKDOWN
    np.testing.assert_array_equal(x, x0)
    # NaN in b -> breakdown, no hang, x0 returned
    bn = b.copy()
    bn[0, 1] = np.nan
    x, it, st, _ = oracle.pcg(x0, S, P, bn, ss, kp, 10, 1e-6, 0.0)
    assert it[0] == 0 and st[0] == oracle.BREAKDOWN
    # warm start from a converged x: the criterion is relative to the new
    # rho_init, so the solve continues from there
    xc, itc, _, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 100, 1e-8, 0.0)
    x2, it2, st2, _ = oracle.pcg(xc, S, P, b, ss, kp, 100, 1e-8, 0.0)
    assert st2[0] == oracle.CONVERGED
    A = oracle.dense_expand(S[0], ss, kp)
    assert np.linalg.norm(b[0] - A @ x2[0]) <= np.linalg.norm(b[0] - A @ xc[0]) * 1.5


def test_pcg_f32_close_to_f64_on_config0():
    """The float32 solve stays within 1e-4 of the float64 solve at equal
    iteration counts (well-conditioned: block-Jacobi kappa ~ 2)."""
    w = workloads.WORKLOADS[0]
    inp = workloads.generate(w, n_problems=16)
    x32, it32, st32, _ = oracle.pcg(inp["x0"], inp["S"], inp["Pinv"], inp["b"],
                                    w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, "f32")
    assert np.all(st32 == oracle.CONVERGED)
    x64, it64, _, _ = oracle.pcg(inp["x0"], inp["S"], inp["Pinv"], inp["b"],
                                 w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, "f64")
    assert np.all(np.abs(it32 - it64) <= 2)
    for q in range(16):
        xf, _, _, _ = oracle.pcg(inp["x0"][q:q + 1], inp["S"][q:q + 1], inp["Pinv"][q:q + 1],
                                 inp["b"][q:q + 1], w.ss, w.kp, int(it32[q]), 0.0, 0.0, "f64")
        rel = np.linalg.norm(x32[q] - xf[0]) / np.linalg.norm(xf[0])
        assert rel <= 1e-4


def test_pcg_threads_bitwise_equal():
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w, n_problems=6)
    a = oracle.pcg(inp["x0"], inp["S"], inp["Pinv"], inp["b"], w.ss, w.kp,
                   w.max_iters, w.rel_tol, w.abs_tol, "f32", nthreads=1)
    b = oracle.pcg(inp["x0"], inp["S"], inp["Pinv"], inp["b"], w.ss, w.kp,
                   w.max_iters, w.rel_tol, w.abs_tol, "f32", nthreads=3)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ---------------------------------------------------------------------------
# bdsv (direct solve)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["bdsv_ss2_kp3.txt", "bdsv_tridiag_ss1_kp5.txt"])
def test_bdsv_golden_hand_examples(name):
    """Systems whose solution was chosen and whose right-hand side was
    multiplied out by hand: catches L/R swapped, a wrong Schur complement
    sign, off-matrix blocks leaking in, or a broken back substitution."""
    g = read_golden(name)
    ss, kp = int(g["ss"][0]), int(g["kp"][0])
    S = frac_array(g["S"]).reshape(1, -1)
    b = frac_array(g["b"]).reshape(1, -1)
    x, st = oracle.bdsv(S, b, ss, kp, "f64")
    assert st[0] == 0
    np.testing.assert_allclose(x[0], frac_array(g["x"]), rtol=0, atol=1e-13)
    x32, st = oracle.bdsv(S.astype(np.float32), b.astype(np.float32), ss, kp, "f32")
    np.testing.assert_allclose(x32[0], frac_array(g["x"]), rtol=0, atol=1e-5)


@pytest.mark.parametrize("embedding", ["ss1", "ss2"])
def test_bdsv_golden_2x2(embedding):
    """A^-1 b = [1/11, 7/11] for the 2x2 system of the CG fixture, in both
    block embeddings."""
    g = read_golden("cg_2x2.txt")
    S, _, ss, kp = _cg2x2_problem(embedding)
    x, st = oracle.bdsv(S, frac_array(g["b"])[None], ss, kp)
    assert st[0] == 0
    np.testing.assert_allclose(x[0], frac_array(g["identity.x2"]), rtol=1e-15, atol=1e-16)


@pytest.mark.parametrize("ss,kp", [(1, 1), (1, 9), (2, 4), (3, 1), (5, 6), (7, 3)])
def test_bdsv_matches_dense_solves(ss, kp):
    """Random SPD systems (the workload recipe) against numpy's LU solve and
    the dense Cholesky solve of the expanded matrix."""
    rng = np.random.default_rng(ss * 31 + kp)
    B = 4
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.2)
    b = rng.standard_normal((B, kp * ss))
    x, st = oracle.bdsv(S, b, ss, kp, nthreads=2)
    assert np.all(st == 0)
    for q in range(B):
        A = oracle.dense_expand(S[q], ss, kp)
        np.testing.assert_allclose(x[q], np.linalg.solve(A, b[q]), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(x[q], oracle.cholesky_solve(A, b[q]), rtol=1e-11, atol=1e-12)


def test_bdsv_symmetric_blocks_from_arbitrary_L():
    """Any symmetric block-tridiagonal SPD matrix (here from random L blocks,
    R_br = L_{br+1}^T, heavy D): catches a Schur complement built with R^T
    where L belongs, or G taken from the wrong block-row."""
    rng = np.random.default_rng(11)
    ss, kp = 3, 5
    L, D, _ = _random_blocks(rng, ss, kp)
    D = D @ np.swapaxes(D, -1, -2) + 12 * np.eye(ss)
    R = np.zeros_like(L)
    R[:-1] = np.swapaxes(L[1:], -1, -2)
    L[0] = 5.0   # off-matrix, must be ignored
    R[-1] = -5.0
    S = _strips_from_blocks(L, D, R)[None]
    b = rng.standard_normal((1, kp * ss))
    x, st = oracle.bdsv(S, b, ss, kp)
    assert st[0] == 0
    L[0] = 0.0
    R[-1] = 0.0
    np.testing.assert_allclose(x[0], np.linalg.solve(_dense_from_blocks(L, D, R), b[0]),
                               rtol=1e-11, atol=1e-12)


def test_bdsv_block_diagonal_and_identity():
    """R = L = 0 decouples into ss x ss solves; D = I returns b."""
    rng = np.random.default_rng(4)
    ss, kp = 4, 3
    S, D = workloads.random_spd_strips(rng, 1, ss, kp, 0.5, offdiag=False)
    b = rng.standard_normal((1, kp * ss))
    x, _ = oracle.bdsv(S, b, ss, kp)
    for br in range(kp):
        np.testing.assert_allclose(x[0, br * ss:(br + 1) * ss],
                                   np.linalg.solve(D[0, br], b[0, br * ss:(br + 1) * ss]),
                                   rtol=1e-12)
    I = workloads.identity_pinv(1, ss, kp)
    x, _ = oracle.bdsv(I, b, ss, kp)
    np.testing.assert_array_equal(x, b)


def test_bdsv_not_spd_status_leaves_x():
    rng = np.random.default_rng(6)
    ss, kp = 3, 4
    S, _ = workloads.random_spd_strips(rng, 2, ss, kp, 0.3)
    S[1] = -S[1]
    b = rng.standard_normal((2, kp * ss))
    x0 = np.full((2, kp * ss), 7.0)
    x, st = oracle.bdsv(S, b, ss, kp, x=x0)
    assert list(st) == [0, 1]
    np.testing.assert_array_equal(x[1], x0[1])


def test_bdsv_agrees_with_converged_pcg():
    """The direct and the iterative solve of the same SPD systems meet."""
    w = workloads.WORKLOADS[0]
    inp = workloads.generate(w, n_problems=6)
    S64, P64, b64 = (inp[k].astype(np.float64) for k in ("S", "Pinv", "b"))
    xd, st = oracle.bdsv(S64, b64, w.ss, w.kp)
    xp, it, _, _ = oracle.pcg(np.zeros_like(b64), S64, P64, b64, w.ss, w.kp, 500, 1e-26, 0.0)
    assert np.all(st == 0)
    np.testing.assert_allclose(xd, xp, rtol=1e-10, atol=1e-12)


def test_bdsv_f32_close_to_f64():
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w, n_problems=4)
    x32, _ = oracle.bdsv(inp["S"], inp["b"], w.ss, w.kp, "f32")
    x64, _ = oracle.bdsv(inp["S"].astype(np.float64), inp["b"].astype(np.float64), w.ss, w.kp)
    rel = np.linalg.norm(x32 - x64, axis=1) / np.linalg.norm(x64, axis=1)
    assert rel.max() < 1e-5


def test_pcg_exact_inverse_in_strip_form_one_iteration():
    """kp = 2: S^-1 is a full 2x2 block matrix, which the [L|D|R] layout holds
    exactly (row 0: [0 | X00 | X01], row 1: [X10 | X11 | 0]).  With Pinv =
    S^-1, z0 = S^-1 r0 = x* - x0, so alpha = 1 and PCG lands on x* after one
    iteration.  A Pinv whose L or R part were read at the wrong place,
    transposed, or dropped would not."""
    rng = np.random.default_rng(123)
    ss, kp, B = 3, 2, 4
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.3)
    P = np.zeros_like(S)
    for q in range(B):
        X = np.linalg.inv(oracle.dense_expand(S[q], ss, kp))
        P[q, 0, :, ss:2 * ss] = X[:ss, :ss]
        P[q, 0, :, 2 * ss:] = X[:ss, ss:]
        P[q, 1, :, :ss] = X[ss:, :ss]
        P[q, 1, :, ss:2 * ss] = X[ss:, ss:]
    b = rng.standard_normal((B, kp * ss))
    x0 = rng.standard_normal((B, kp * ss))
    x, it, st, _ = oracle.pcg(x0, S, P, b, ss, kp, 10, 1e-20, 0.0)
    assert np.all(it == 1) and np.all(st == oracle.CONVERGED), (it, st)
    for q in range(B):
        A = oracle.dense_expand(S[q], ss, kp)
        np.testing.assert_allclose(x[q], np.linalg.solve(A, b[q]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("ss,kp", [(2, 4), (5, 6)])
def test_pcg_block_tridiagonal_pinv_matches_dense_solve(ss, kp):
    """With the SPD block-tridiagonal preconditioner of the generator (non-zero
    L/R blocks), PCG converges to the dense solution, in no more iterations
    than with block Jacobi (a better preconditioner: Pinv S ~ I - F^2)."""
    rng = np.random.default_rng(ss * 5 + kp)
    B = 4
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2)
    P = workloads.block_tridiagonal_pinv(S, D)
    Pj = workloads.block_jacobi_pinv(D)
    b = rng.standard_normal((B, kp * ss))
    x, it, st, _ = oracle.pcg(np.zeros_like(b), S, P, b, ss, kp, 100, 1e-26, 0.0)
    _, itj, _, _ = oracle.pcg(np.zeros_like(b), S, Pj, b, ss, kp, 100, 1e-26, 0.0)
    assert np.all(st == oracle.CONVERGED)
    assert np.all(it <= itj), (it, itj)
    for q in range(B):
        A = oracle.dense_expand(S[q], ss, kp)
        np.testing.assert_allclose(x[q], np.linalg.solve(A, b[q]), rtol=1e-10, atol=1e-12)
