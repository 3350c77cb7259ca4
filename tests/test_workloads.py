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
