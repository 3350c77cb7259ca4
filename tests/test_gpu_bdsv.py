"""GPU parity of glass_bdsv_batched (direct block-tridiagonal SPD solve)
against the CPU oracle through the C ABI.

Bar: the solution of an SPD system is unique, so x is compared with the
float64 oracle solution: relative L2 error <= 1e-4 (float32) / 1e-10
(float64).  The forward error of a stable direct solve is about
cond(A) * n * eps: the workload matrices have cond(A) of order 10, which
puts float32 errors near 1e-6 and float64 near 1e-14."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import frac_array, read_golden
from gpu_common import X_REL, pcg_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def bdsv_gpu(glass, S, b, ss, kp, x0=None):
    St, bt = to_dev(S), to_dev(b)
    x = to_dev(np.full(b.shape, np.nan, b.dtype) if x0 is None else x0).clone()
    st = torch.full((b.shape[0],), -1, dtype=torch.int32, device="cuda")
    glass.bdsv_batched(x, St, bt, ss, kp, st)
    torch.cuda.synchronize()
    return x.cpu().numpy(), st.cpu().numpy()


def assert_bdsv_parity(S, b, ss, kp, x, st, dtype):
    xr, sr = oracle.bdsv(np.asarray(S, np.float64), np.asarray(b, np.float64), ss, kp,
                         "f64", nthreads=8)
    np.testing.assert_array_equal(st, sr)
    ok = sr == 0
    num = np.linalg.norm(x[ok].astype(np.float64) - xr[ok], axis=1)
    den = np.maximum(np.linalg.norm(xr[ok], axis=1), 1e-300)
    worst = float((num / den).max()) if ok.any() else 0.0
    assert worst <= X_REL[dtype], "x relative L2 error %g" % worst


@pytest.mark.parametrize("cfg,B", [(0, 64), (2, 33), (3, 9)])
def test_bdsv_workload_shapes(gpu, cfg, B):
    w = workloads.CONFIGS[cfg]
    inp = workloads.generate(w, n_problems=B)
    say("bdsv cfg%d shape ss=%d kp=%d B=%d" % (cfg, w.ss, w.kp, B))
    x, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(inp["S"], inp["b"], w.ss, w.kp, x, st, np.float32)


def test_bdsv_full_batch_ss14(gpu):
    """All 4096 systems of the ss=14, kp=32 workload, every x checked."""
    w = workloads.CONFIGS[2]
    inp = workloads.generate(w)
    say("bdsv full ss=14 kp=32 B=4096")
    x, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(inp["S"], inp["b"], w.ss, w.kp, x, st, np.float32)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("ss,kp,B", [(1, 1, 3), (1, 300, 2), (2, 5, 4), (5, 1, 3),
                                     (7, 40, 3), (12, 64, 2), (16, 20, 2), (24, 12, 2)])
def test_bdsv_edge_shapes(gpu, ss, kp, B, dtype):
    rng = np.random.default_rng(ss * 1000 + kp)
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.2, dtype)
    S[:, 0, :, :ss] = 3.0        # off-matrix blocks are ignored
    S[:, -1, :, 2 * ss:] = -3.0
    b = rng.standard_normal((B, kp * ss)).astype(dtype)
    say("bdsv ss=%d kp=%d B=%d %s" % (ss, kp, B, np.dtype(dtype).name))
    x, st = bdsv_gpu(gpu, S, b, ss, kp)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(S, b, ss, kp, x, st, dtype)


@pytest.mark.parametrize("name", ["bdsv_ss2_kp3.txt", "bdsv_tridiag_ss1_kp5.txt"])
def test_bdsv_golden_fixtures(gpu, name):
    g = read_golden(name)
    ss, kp = int(g["ss"][0]), int(g["kp"][0])
    S = frac_array(g["S"]).reshape(1, -1)
    b = frac_array(g["b"]).reshape(1, -1)
    say("bdsv golden %s" % name)
    x, st = bdsv_gpu(gpu, S, b, ss, kp)
    assert st[0] == gpu.BDSV_OK
    np.testing.assert_allclose(x[0], frac_array(g["x"]), rtol=0, atol=1e-12)


def test_bdsv_not_spd_leaves_x_and_flags(gpu):
    rng = np.random.default_rng(12)
    ss, kp, B = 6, 10, 4
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.3, np.float32)
    S[1] = -S[1]
    S[3, 4, :, ss:2 * ss] = 0.0   # a singular diagonal block mid-chain
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    x0 = np.full((B, kp * ss), 5.0, np.float32)
    say("bdsv status cases")
    x, st = bdsv_gpu(gpu, S, b, ss, kp, x0=x0)
    _, so = oracle.bdsv(S, b, ss, kp, "f32")
    np.testing.assert_array_equal(st, so)
    assert st[1] == gpu.BDSV_NOT_SPD and st[0] == gpu.BDSV_OK
    np.testing.assert_array_equal(x[1], x0[1])
    assert_bdsv_parity(S[[0, 2]], b[[0, 2]], ss, kp, x[[0, 2]], st[[0, 2]], np.float32)


def test_bdsv_agrees_with_gpu_pcg_and_is_deterministic(gpu):
    """The direct solve meets the GPU's PCG solution to PCG's own accuracy,
    and repeats bit for bit."""
    w = workloads.CONFIGS[0]
    inp = workloads.generate(w)
    say("bdsv vs pcg")
    x1, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    x2, _ = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    np.testing.assert_array_equal(x1, x2)
    xp, it, sp, _ = pcg_gpu(gpu, inp, w.ss, w.kp, 500, 1e-12, 0.0)
    rel = np.linalg.norm(x1 - xp, axis=1) / np.linalg.norm(x1, axis=1)
    assert rel.max() < 1e-4


def test_bdsv_lds_limit_is_reported(gpu):
    S = torch.zeros(24 * 3 * 24 * 100, dtype=torch.float32, device="cuda")
    b = torch.zeros(24 * 100, dtype=torch.float32, device="cuda")
    x = torch.zeros_like(b)
    with pytest.raises(gpu.GlassError) as ei:
        gpu.bdsv_batched(x, S, b, 24, 100)
    assert ei.value.code == -2
