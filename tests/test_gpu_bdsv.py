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


@pytest.fixture(params=["rows", "columns"])
def mapping(request, monkeypatch):
    """The two kernel mappings: four problems per wave with one row of W per
    lane (state sizes up to 16), or one problem per wave with one column per
    lane (forced here with GLASS_AMD_BDSV_COLUMNS)."""
    if request.param == "columns":
        monkeypatch.setenv("GLASS_AMD_BDSV_COLUMNS", "1")
    else:
        monkeypatch.delenv("GLASS_AMD_BDSV_COLUMNS", raising=False)
    return request.param


def bdsv_gpu(glass, S, b, ss, kp, x0=None, ws=False):
    """ws: keep the per-block-row factors in a workspace in HBM instead of
    LDS (the two placements must agree bit for bit)."""
    St, bt = to_dev(S), to_dev(b)
    x = to_dev(np.full(b.shape, np.nan, b.dtype) if x0 is None else x0).clone()
    st = torch.full((b.shape[0],), -1, dtype=torch.int32, device="cuda")
    work = None
    if ws:
        nbytes = glass.bdsv_workspace_bytes(ss, kp, b.shape[0], St.dtype)
        work = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    glass.bdsv_batched(x, St, bt, ss, kp, st, workspace=work)
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


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("cfg,B", [(0, 64), (2, 33), (3, 9)])
def test_bdsv_workload_shapes(gpu, cfg, B, ws, mapping):
    w = workloads.WORKLOADS[cfg]
    inp = workloads.generate(w, n_problems=B)
    say("bdsv cfg%d shape ss=%d kp=%d B=%d ws=%s %s" % (cfg, w.ss, w.kp, B, ws, mapping))
    x, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp, ws=ws)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(inp["S"], inp["b"], w.ss, w.kp, x, st, np.float32)


def test_bdsv_full_batch_ss14_both_placements(gpu):
    """All 4096 systems of the ss=14, kp=32 workload, every x checked; the
    LDS and the workspace placements give the same bits."""
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w)
    say("bdsv full ss=14 kp=32 B=4096")
    x, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(inp["S"], inp["b"], w.ss, w.kp, x, st, np.float32)
    x2, st2 = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp, ws=True)
    np.testing.assert_array_equal(st2, st)
    np.testing.assert_array_equal(x2, x)


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("ss,kp,B", [(1, 1, 3), (1, 300, 2), (2, 5, 4), (5, 1, 3),
                                     (7, 40, 3), (12, 64, 2), (16, 20, 2), (24, 12, 2),
                                     (13, 7, 3), (6, 10, 7), (14, 3, 5), (16, 9, 9),
                                     (3, 2, 1)])
def test_bdsv_edge_shapes(gpu, ss, kp, B, dtype, ws, mapping):
    rng = np.random.default_rng(ss * 1000 + kp)
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.2, dtype)
    S[:, 0, :, :ss] = 3.0        # off-matrix blocks are ignored
    S[:, -1, :, 2 * ss:] = -3.0
    b = rng.standard_normal((B, kp * ss)).astype(dtype)
    say("bdsv ss=%d kp=%d B=%d %s ws=%s %s" % (ss, kp, B, np.dtype(dtype).name, ws, mapping))
    x, st = bdsv_gpu(gpu, S, b, ss, kp, ws=ws)
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


@pytest.mark.parametrize("ws", [False, True])
def test_bdsv_not_spd_leaves_x_and_flags(gpu, ws, mapping):
    rng = np.random.default_rng(12)
    ss, kp, B = 6, 10, 4
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.3, np.float32)
    S[1] = -S[1]
    S[3, 4, :, ss:2 * ss] = 0.0   # a singular diagonal block mid-chain
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    x0 = np.full((B, kp * ss), 5.0, np.float32)
    say("bdsv status cases ws=%s %s" % (ws, mapping))
    x, st = bdsv_gpu(gpu, S, b, ss, kp, x0=x0, ws=ws)
    _, so = oracle.bdsv(S, b, ss, kp, "f32")
    np.testing.assert_array_equal(st, so)
    assert st[1] == gpu.BDSV_NOT_SPD and st[0] == gpu.BDSV_OK
    np.testing.assert_array_equal(x[1], x0[1])
    assert_bdsv_parity(S[[0, 2]], b[[0, 2]], ss, kp, x[[0, 2]], st[[0, 2]], np.float32)


def test_bdsv_agrees_with_gpu_pcg_and_is_deterministic(gpu):
    """The direct solve meets the GPU's PCG solution to PCG's own accuracy,
    and repeats bit for bit."""
    w = workloads.WORKLOADS[0]
    inp = workloads.generate(w)
    say("bdsv vs pcg")
    x1, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    x2, _ = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp)
    np.testing.assert_array_equal(x1, x2)
    xp, it, sp, _ = pcg_gpu(gpu, inp, w.ss, w.kp, 500, 1e-12, 0.0)
    rel = np.linalg.norm(x1 - xp, axis=1) / np.linalg.norm(x1, axis=1)
    assert rel.max() < 1e-4


def test_bdsv_lds_limit_is_reported_and_the_workspace_lifts_it(gpu):
    """ss=24, kp=100: the factors (240 KB per problem) exceed LDS; with a
    workspace the chain solves."""
    rng = np.random.default_rng(21)
    ss, kp, B = 24, 100, 2
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.2, np.float32)
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    St, bt = to_dev(S), to_dev(b)
    x = torch.zeros_like(bt)
    with pytest.raises(gpu.GlassError) as ei:
        gpu.bdsv_batched(x, St, bt, ss, kp)
    assert ei.value.code == -2
    say("bdsv long chain with workspace")
    xg, st = bdsv_gpu(gpu, S, b, ss, kp, ws=True)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(S, b, ss, kp, xg, st, np.float32)


def test_bdsv_rows_and_columns_meet_the_oracle_on_the_full_batch(gpu, monkeypatch):
    """Both mappings on all 4096 ss=14 kp=32 systems, each against the
    oracle (they round differently, so they are not compared bit for bit)."""
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w)
    for cols in ("0", "1"):
        monkeypatch.setenv("GLASS_AMD_BDSV_COLUMNS", cols)
        say("bdsv full ss=14 kp=32 columns=%s" % cols)
        x, st = bdsv_gpu(gpu, inp["S"], inp["b"], w.ss, w.kp, ws=True)
        assert np.all(st == gpu.BDSV_OK)
        assert_bdsv_parity(inp["S"], inp["b"], w.ss, w.kp, x, st, np.float32)


def test_bdsv_long_chain_without_workspace_uses_the_column_mapping(gpu):
    """ss=14, kp=100 without a workspace: four problems' factors (336 KB)
    do not fit in LDS for the row mapping, one problem's (84 KB) do, so the
    solve runs (column mapping) and meets the oracle."""
    rng = np.random.default_rng(31)
    ss, kp, B = 14, 100, 5
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.2, np.float32)
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    say("bdsv ss=14 kp=100 no workspace")
    x, st = bdsv_gpu(gpu, S, b, ss, kp)
    assert np.all(st == gpu.BDSV_OK)
    assert_bdsv_parity(S, b, ss, kp, x, st, np.float32)
