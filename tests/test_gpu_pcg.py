"""GPU parity of glass_pcg_batched against the CPU oracle through the C ABI.
Bars (see gpu_common): iterations within +-2, x within 1e-4 (fp32) / 1e-10
(fp64) relative L2 of the oracle at the same iteration count, final criterion
met."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import assert_pcg_parity, pack_diagonal_blocks, pcg_gpu, say

pytestmark = pytest.mark.gpu


def run_workload(gpu, cfg, n_problems=None, dtype=None):
    w = workloads.WORKLOADS[cfg]
    inp = workloads.generate(w, n_problems=n_problems)
    if dtype is not None:
        inp = {k: v.astype(dtype) for k, v in inp.items()}
    dt = inp["b"].dtype.type
    say("pcg cfg%d B=%d %s" % (cfg, inp["b"].shape[0], np.dtype(dt).name))
    res = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    assert np.all(res[2] == gpu.CONVERGED)
    return assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, res, dt)


@pytest.mark.parametrize("cfg", [0, 2, 3])
def test_pcg_workloads_reduced_batch(gpu, cfg):
    run_workload(gpu, cfg, n_problems=33)


@pytest.mark.parametrize("cfg", [0, 2, 3])
def test_pcg_workloads_full_batch(gpu, cfg):
    its = run_workload(gpu, cfg)
    say("  iterations: %s" % dict(zip(*np.unique(its, return_counts=True))))


@pytest.mark.parametrize("cfg", [0, 2, 3])
def test_pcg_fp64(gpu, cfg):
    run_workload(gpu, cfg, n_problems=17, dtype=np.float64)


def test_pcg_placements_bit_identical(gpu, monkeypatch):
    """Thread-count invariance: the dots add fixed 64-row chunk partials in
    chunk order and every row is contracted serially in index order, so the
    register-resident placement and the streamed placements at 1, 2, 3, 4
    and 8 rows per lane (1 to 7 waves) give the same bits."""
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w, n_problems=24)
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, ref, np.float32)
    monkeypatch.setenv("GLASS_AMD_PCG_STREAMED", "1")
    for rpt in ("1", "2", "3", "4", "8"):
        for pf in ("0", "1"):
            monkeypatch.setenv("GLASS_AMD_PCG_RPT", rpt)
            if pf == "0":
                monkeypatch.setenv("GLASS_AMD_PCG_NO_PREFETCH", "1")
            else:
                monkeypatch.delenv("GLASS_AMD_PCG_NO_PREFETCH", raising=False)
            say("pcg cfg2 streamed rows/lane=%s prefetch=%s" % (rpt, pf))
            got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
            for u, v in zip(ref, got):
                np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("ss,kp,B,margin,dtype", [
    (1, 1, 4, 0.5, np.float32), (1, 700, 3, 0.3, np.float32),
    (2, 4, 5, 0.3, np.float32), (5, 9, 6, 0.2, np.float32),
    (6, 1, 3, 0.5, np.float32), (7, 150, 3, 0.2, np.float32),
    (14, 50, 4, 0.2, np.float32), (33, 10, 2, 0.2, np.float32),
    (64, 5, 2, 0.3, np.float32),
    # streamed with the two-deep prefetch ring: 1, 2, 4 and 8 chunks per
    # wave, ragged last chunks, and float64
    (21, 20, 3, 0.1, np.float32), (21, 40, 2, 0.1, np.float32),
    (6, 200, 2, 0.3, np.float32), (12, 300, 2, 0.2, np.float32),
    (21, 100, 1, 0.1, np.float32), (6, 200, 2, 0.3, np.float64),
])
def test_pcg_generic_shapes(gpu, ss, kp, B, margin, dtype):
    """Specialised and runtime state sizes, ragged last chunk, kp = 1, several
    rows per lane (n up to 3600), resident and streamed placements."""
    rng = np.random.default_rng(ss * 100 + kp)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, margin, dtype)
    inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
           "b": rng.standard_normal((B, kp * ss)).astype(dtype),
           "x0": np.zeros((B, kp * ss), dtype)}
    rel = 1e-8 if dtype == np.float32 else 1e-14
    say("pcg ss=%d kp=%d B=%d %s" % (ss, kp, B, np.dtype(dtype).name))
    res = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, res, dtype)


def test_pcg_nonzero_initial_guess_and_block_tridiagonal_pinv(gpu):
    """x0 != 0 and a Pinv with non-zero L/R blocks (the kernels treat Pinv as a
    general [L|D|R] matrix)."""
    rng = np.random.default_rng(3)
    ss, kp, B = 6, 32, 16
    S, _ = workloads.random_spd_strips(rng, B, ss, kp, 0.5, np.float64)
    P, _ = workloads.random_spd_strips(rng, B, ss, kp, 3.0, np.float64)
    P = P / 8.0
    inp = {"S": S.astype(np.float32), "Pinv": P.astype(np.float32),
           "b": rng.standard_normal((B, kp * ss)).astype(np.float32),
           "x0": rng.standard_normal((B, kp * ss)).astype(np.float32)}
    say("pcg x0!=0, tridiagonal Pinv")
    res = pcg_gpu(gpu, inp, ss, kp, 200, 1e-7, 0.0)
    assert np.all(res[2] == gpu.CONVERGED)
    assert_pcg_parity(inp, ss, kp, 200, 1e-7, 0.0, res, np.float32)


def test_pcg_status_cases(gpu):
    rng = np.random.default_rng(8)
    ss, kp, B = 6, 8, 6
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.5, np.float32)
    P = workloads.block_jacobi_pinv(D, np.float32)
    b = rng.standard_normal((B, kp * ss)).astype(np.float32)
    x0 = rng.standard_normal((B, kp * ss)).astype(np.float32)
    S[1] = -S[1]            # negative definite -> breakdown at the first step
    b[2] = 0.0              # with x0 = 0 below: rho_init == 0 -> converged, 0 its
    b[3, 5] = np.nan        # NaN -> breakdown, no hang
    x0[2] = 0.0
    inp = {"S": S, "Pinv": P, "b": b, "x0": x0}
    say("pcg status cases")
    x, it, st, rho = pcg_gpu(gpu, inp, ss, kp, 50, 1e-6, 0.0)
    xo, ito, sto, rhoo = oracle.pcg(x0, S, P, b, ss, kp, 50, 1e-6, 0.0, "f32")
    np.testing.assert_array_equal(st, sto)
    assert st[1] == gpu.BREAKDOWN and it[1] == 0
    assert st[2] == gpu.CONVERGED and it[2] == 0 and np.all(x[2] == 0)
    assert st[3] == gpu.BREAKDOWN and it[3] == 0
    assert np.all(np.abs(it - ito) <= 2)
    # max_iters = 0 and a huge abs_tol
    x, it, st, _ = pcg_gpu(gpu, inp, ss, kp, 0, 1e-6, 0.0)
    assert np.all(it == 0)
    assert st[0] == gpu.MAX_ITERS
    np.testing.assert_array_equal(x[0], x0[0])
    x, it, st, _ = pcg_gpu(gpu, inp, ss, kp, 50, 0.0, 1e30)
    assert np.all(it == 0) and np.all(st[[0, 2, 4, 5]] == gpu.CONVERGED)


def test_pcg_max_iters_exhausted(gpu):
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w, n_problems=8)
    say("pcg max_iters=2")
    res = pcg_gpu(gpu, inp, w.ss, w.kp, 2, w.rel_tol, w.abs_tol)
    assert np.all(res[1] == 2) and np.all(res[2] == gpu.MAX_ITERS)
    assert_pcg_parity(inp, w.ss, w.kp, 2, w.rel_tol, w.abs_tol, res, np.float32)


def test_pcg_run_to_run_deterministic(gpu):
    w = workloads.WORKLOADS[3]
    inp = workloads.generate(w, n_problems=12)
    a = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    b = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_pcg_rejects_inconsistent_buffers(gpu):
    w = workloads.WORKLOADS[0]
    inp = workloads.generate(w, n_problems=2)
    t = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    it = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        gpu.pcg_batched(t["x0"][:1], t["S"], t["Pinv"], t["b"], w.ss, w.kp, 10, 1e-6, 0.0, it)
    with pytest.raises(TypeError):
        gpu.pcg_batched(t["x0"], t["S"], t["Pinv"], t["b"], w.ss, w.kp, 10, 1e-6, 0.0,
                        it.to(torch.int64))


def test_pcg_prefetch_ring_matches_plain_staging(gpu, monkeypatch):
    """The prefetching and the plain streamed placements stage the same bytes
    and run the same arithmetic in the same order: bit-identical outputs."""
    w = workloads.WORKLOADS[3]
    inp = workloads.generate(w, n_problems=10)
    say("pcg cfg3 prefetch vs plain staging")
    monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
    a = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    monkeypatch.setenv("GLASS_AMD_PCG_NO_PREFETCH", "1")
    b = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_pcg_placement_query_matches_the_workloads(gpu, monkeypatch):
    """S and Pinv stay in registers for the ss=6 and ss=14 fp32 workloads; for
    ss=21 kp=64 S stays in registers and Pinv streams (with prefetch when the
    S-resident placement is switched off); forcing streaming is reported."""
    assert gpu.pcg_batched_placement(6, 32, torch.float32) == gpu.PLACEMENT_RESIDENT
    assert gpu.pcg_batched_placement(14, 32, torch.float32) == gpu.PLACEMENT_RESIDENT
    assert gpu.pcg_batched_placement(21, 64, torch.float32) == gpu.PLACEMENT_S_RESIDENT
    assert gpu.pcg_batched_placement(14, 32, torch.float64) == gpu.PLACEMENT_S_RESIDENT
    # element-aligned matrices keep S in registers at ss=21 (shifted chunk loads)
    assert gpu.pcg_batched_placement(21, 64, torch.float32, aligned16=False) == \
        gpu.PLACEMENT_S_RESIDENT
    assert gpu.pcg_batched_placement(21, 64, torch.float32, aligned16=False,
                                      pinv_block_diagonal=True) == gpu.PLACEMENT_STREAMED
    assert gpu.pcg_batched_placement(21, 64, torch.float32, pinv_block_diagonal=True) == \
        gpu.PLACEMENT_RESIDENT
    # ss=21 kp=64 (21 chunks of 64 rows, 3 per wave): with 8 waves, the LDS
    # left over pins the last chunk of wave 0, and waves 5-7, which have no
    # third chunk, hold their chunk 0 of Pinv in those registers: 4 chunks.
    assert gpu.pcg_batched_pinned_rows(21, 64, torch.float32) == 256
    # kp=40 (14 chunks, 2 per wave, 8 waves): one LDS slot, waves 6 and 7
    assert gpu.pcg_batched_pinned_rows(21, 40, torch.float32) == 192
    assert gpu.pcg_batched_pinned_rows(14, 32, torch.float64) == 0  # one row per lane
    assert gpu.pcg_batched_pinned_rows(14, 32, torch.float32) == 0  # resident
    monkeypatch.setenv("GLASS_AMD_PCG_NO_PIN", "1")
    assert gpu.pcg_batched_pinned_rows(21, 64, torch.float32) == 0
    monkeypatch.delenv("GLASS_AMD_PCG_NO_PIN")
    monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
    assert gpu.pcg_batched_placement(21, 64, torch.float32, pinv_block_diagonal=True) == \
        gpu.PLACEMENT_STREAMED_PREFETCH
    assert gpu.pcg_batched_placement(21, 64, torch.float32) == gpu.PLACEMENT_STREAMED_PREFETCH
    monkeypatch.delenv("GLASS_AMD_PCG_NO_HYBRID")
    monkeypatch.setenv("GLASS_AMD_PCG_STREAMED", "1")
    assert gpu.pcg_batched_placement(21, 64, torch.float32) == gpu.PLACEMENT_STREAMED_PREFETCH
    assert gpu.pcg_batched_placement(14, 32, torch.float32) != gpu.PLACEMENT_RESIDENT
    with pytest.raises(gpu.GlassError):
        gpu.pcg_batched_placement(64, 200, torch.float32)


def test_pcg_full_batch_fp64_variant(gpu):
    """The float64 variant of the ss=14 workload at the size bench.py times
    (4096 problems), every x checked against the float64 oracle."""
    run_workload(gpu, 2, dtype=np.float64)


@pytest.mark.parametrize("ss,kp,fits", [(6, 1365, True), (12, 340, True), (12, 682, False),
                                         (21, 195, True), (21, 390, False)])
def test_pcg_largest_batched_rows(gpu, ss, kp, fits):
    """Near the row limit of one workgroup: the streamed placement holds a
    64-row LDS stage per wave, so wide rows cap the rows per problem below
    8192 (ss=12: 16 waves x 8 rows per lane need more than 160 KB of LDS).
    Shapes that fit solve to the parity bar; the others are refused with
    GLASS_EUNSUPPORTED before anything is launched."""
    rng = np.random.default_rng(ss + kp)
    B = 2
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2, np.float32)
    inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, np.float32),
           "b": rng.standard_normal((B, kp * ss)).astype(np.float32),
           "x0": np.zeros((B, kp * ss), np.float32)}
    say("pcg ss=%d kp=%d (n=%d)" % (ss, kp, ss * kp))
    if not fits:
        with pytest.raises(gpu.GlassError) as ei:
            gpu.pcg_batched_placement(ss, kp, torch.float32)
        assert ei.value.code == -2
        with pytest.raises(gpu.GlassError) as ei:
            pcg_gpu(gpu, inp, ss, kp, 300, 1e-8, 0.0)
        assert ei.value.code == -2
        return
    res = pcg_gpu(gpu, inp, ss, kp, 300, 1e-8, 0.0)
    assert_pcg_parity(inp, ss, kp, 300, 1e-8, 0.0, res, np.float32)


def test_empty_batches_are_no_ops(gpu):
    z = torch.zeros(0, dtype=torch.float32, device="cuda")
    zi = torch.zeros(0, dtype=torch.int32, device="cuda")
    gpu.pcg_batched(z, z, z, z, 6, 32, 10, 1e-6, 0.0, zi)
    gpu.pcg_batched(z, z, z, z, 6, 32, 10, 1e-6, 0.0, zi, pinv_diagonal_blocks=True)
    gpu.bdsv_batched(z, z, z, 6, 32, zi)
    torch.cuda.synchronize()


@pytest.mark.parametrize("ss,kp,B,dtype,resident_only_with_flag", [
    (14, 32, 96, np.float32, False),   # the resident ss=14 workload shape
    (6, 32, 40, np.float32, False),
    (12, 60, 9, np.float32, False),
    (21, 40, 7, np.float32, True),     # 840 rows: resident only with the flag
    (6, 20, 9, np.float64, False),
    (21, 64, 5, np.float32, True),     # S resident; with the flag the D parts in LDS too
])
def test_pcg_pinv_block_diagonal_hint(gpu, ss, kp, B, dtype, resident_only_with_flag):
    """GLASS_PCG_PINV_BLOCK_DIAGONAL on block-Jacobi preconditioners: the
    same values as the general contraction (the skipped terms are exact
    zeros added in the same order) and oracle parity; the placement query
    reports where the rows go."""
    rng = np.random.default_rng(ss * 100 + kp)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2, dtype)
    inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
           "b": rng.standard_normal((B, kp * ss)).astype(dtype),
           "x0": np.zeros((B, kp * ss), dtype)}
    rel = 1e-6 if dtype == np.float32 else 1e-10
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    plain = gpu.pcg_batched_placement(ss, kp, tdt)
    hinted = gpu.pcg_batched_placement(ss, kp, tdt, pinv_block_diagonal=True)
    if resident_only_with_flag:
        assert plain != gpu.PLACEMENT_RESIDENT and hinted == gpu.PLACEMENT_RESIDENT
    elif plain == gpu.PLACEMENT_RESIDENT:
        assert hinted == gpu.PLACEMENT_RESIDENT
    say("pcg Pinv block-diagonal ss=%d kp=%d B=%d %s placement %d -> %d"
        % (ss, kp, B, np.dtype(dtype).name, plain, hinted))
    ref = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
    got = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0, pinv_block_diagonal=True)
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, got, dtype)


def test_pcg_pinv_block_diagonal_full_workload(gpu):
    """The full 4096-problem ss=14 workload with the hint, against the
    general run and the oracle."""
    w = workloads.WORKLOADS[2]
    inp = workloads.generate(w)
    say("pcg cfg2 full with the block-diagonal Pinv hint")
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                  pinv_block_diagonal=True)
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)


def test_pcg_pinv_block_diagonal_streamed_prefetch(gpu, monkeypatch):
    """The streamed placement with prefetch fetches only the Pinv vectors
    that touch a D block under the hint: the same values as the general run
    for the full ss=21 workload, and at 1, 2 and 4 rows per lane for ss=14."""
    w = workloads.WORKLOADS[3]
    inp = workloads.generate(w)
    say("pcg cfg3 full with the block-diagonal Pinv hint")
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                  pinv_block_diagonal=True)
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)
    w2 = workloads.WORKLOADS[2]
    inp2 = workloads.generate(w2, n_problems=20)
    monkeypatch.setenv("GLASS_AMD_PCG_STREAMED", "1")
    for rpt in ("1", "2", "4"):
        monkeypatch.setenv("GLASS_AMD_PCG_RPT", rpt)
        say("pcg cfg2 streamed prefetch rows/lane=%s with the hint" % rpt)
        ref = pcg_gpu(gpu, inp2, w2.ss, w2.kp, w2.max_iters, w2.rel_tol, w2.abs_tol)
        got = pcg_gpu(gpu, inp2, w2.ss, w2.kp, w2.max_iters, w2.rel_tol, w2.abs_tol,
                      pinv_block_diagonal=True)
        for u, v in zip(ref, got):
            np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("ss,kp,B,dtype", [
    (14, 32, 96, np.float32),   # resident (D blocks only)
    (6, 32, 40, np.float32),
    (12, 60, 9, np.float32),
    (21, 40, 7, np.float32),    # 840 rows: resident with D blocks
    (21, 64, 5, np.float32),    # S in registers, D blocks in LDS
    (6, 20, 9, np.float64),
    (14, 32, 6, np.float64),    # S in registers, D blocks in LDS
    (14, 100, 3, np.float64),   # plain streamed staging, specialised size
    (9, 32, 5, np.float32),     # plain streamed staging, generic size, 16-byte paths
    (9, 23, 5, np.float32),     # generic size, ragged last chunk, element paths
    (14, 1, 3, np.float32),     # one block-row (Pinv is exactly inv(S))
    (21, 2, 4, np.float32),     # two block-rows
])
def test_pcg_pinv_packed_diagonal_blocks(gpu, ss, kp, B, dtype):
    """GLASS_PCG_PINV_DIAGONAL_BLOCKS: Pinv passed as packed D blocks
    [B, kp, ss, ss] gives the same bits as the [L|D|R] layout with zero L
    and R blocks (the same terms in the same order) in every placement, and
    meets the oracle; the placement query reports the hinted placement, or
    the resident one where S fits in registers and the D blocks in LDS."""
    rng = np.random.default_rng(ss * 1000 + kp)
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2, dtype)
    inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
           "b": rng.standard_normal((B, kp * ss)).astype(dtype),
           "x0": np.zeros((B, kp * ss), dtype)}
    rel = 1e-6 if dtype == np.float32 else 1e-10
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    hinted = gpu.pcg_batched_placement(ss, kp, tdt, pinv_block_diagonal=True)
    packed = gpu.pcg_batched_placement(ss, kp, tdt, pinv_diagonal_blocks=True)
    assert packed == hinted or (packed == gpu.PLACEMENT_RESIDENT
                                and hinted != gpu.PLACEMENT_RESIDENT)
    say("pcg Pinv packed D blocks ss=%d kp=%d B=%d %s placement %d"
        % (ss, kp, B, np.dtype(dtype).name, packed))
    ref = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
    got = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0, pinv_diagonal_blocks=True)
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, got, dtype)


@pytest.mark.parametrize("cfg", [2, 3])
def test_pcg_pinv_packed_element_aligned_pointer(gpu, cfg):
    """Packed D blocks at an address aligned to the element size only: the
    element-load paths (the 16-byte ones need 16-byte alignment) give the
    same bits as the aligned call."""
    w = workloads.WORKLOADS[cfg]
    inp = workloads.generate(w, n_problems=24)
    B = inp["b"].shape[0]
    packed = pack_diagonal_blocks(inp["Pinv"], w.ss, w.kp)
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                  pinv_diagonal_blocks=True)
    store = torch.zeros(packed.size + 1, dtype=torch.float32, device="cuda")
    P = store[1:]
    P.copy_(torch.from_numpy(packed.reshape(-1)))
    assert P.data_ptr() % 16 == 4
    x = torch.from_numpy(inp["x0"]).cuda()
    it = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    st = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, 2), dtype=torch.float32, device="cuda")
    say("pcg cfg%d packed Pinv at a 4-byte-aligned address" % cfg)
    gpu.pcg_batched(x, torch.from_numpy(inp["S"]).cuda(), P, torch.from_numpy(inp["b"]).cuda(),
                    w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, it, st, rho,
                    pinv_diagonal_blocks=True)
    torch.cuda.synchronize()
    got = (x.cpu().numpy(), it.cpu().numpy(), st.cpu().numpy(), rho.cpu().numpy())
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)


def test_pcg_pinv_packed_diagonal_blocks_workloads(gpu, monkeypatch):
    """Packed D blocks on both full workloads (ss=14 resident, ss=21 with S
    in registers and the D blocks in LDS) against the [L|D|R] runs, then the other
    streamed forms: prefetch at 1, 2 and 4 rows per lane, and plain
    staging."""
    for cfg in (2, 3):
        w = workloads.WORKLOADS[cfg]
        inp = workloads.generate(w)
        say("pcg cfg%d full with packed Pinv D blocks" % cfg)
        ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
        got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                      pinv_diagonal_blocks=True)
        for u, v in zip(ref, got):
            np.testing.assert_array_equal(u, v)
        assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)
    w2 = workloads.WORKLOADS[2]
    inp2 = workloads.generate(w2, n_problems=20)
    ref2 = pcg_gpu(gpu, inp2, w2.ss, w2.kp, w2.max_iters, w2.rel_tol, w2.abs_tol)
    monkeypatch.setenv("GLASS_AMD_PCG_STREAMED", "1")
    assert gpu.pcg_batched_placement(w2.ss, w2.kp, torch.float32, pinv_diagonal_blocks=True) \
        == gpu.PLACEMENT_STREAMED_PREFETCH
    for rpt in ("1", "2", "4"):
        monkeypatch.setenv("GLASS_AMD_PCG_RPT", rpt)
        say("pcg cfg2 streamed prefetch rows/lane=%s, packed Pinv D blocks" % rpt)
        got = pcg_gpu(gpu, inp2, w2.ss, w2.kp, w2.max_iters, w2.rel_tol, w2.abs_tol,
                      pinv_diagonal_blocks=True)
        for u, v in zip(ref2, got):
            np.testing.assert_array_equal(u, v)
    monkeypatch.delenv("GLASS_AMD_PCG_RPT")
    monkeypatch.setenv("GLASS_AMD_PCG_NO_PREFETCH", "1")
    monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")  # ss=21: plain staging too
    assert gpu.pcg_batched_placement(w2.ss, w2.kp, torch.float32, pinv_diagonal_blocks=True) \
        == gpu.PLACEMENT_STREAMED
    w3 = workloads.WORKLOADS[3]
    inp3 = workloads.generate(w3, n_problems=12)
    for w, inp, ref in ((w2, inp2, ref2), (w3, inp3, None)):
        say("pcg ss=%d plain streamed staging, packed Pinv D blocks" % w.ss)
        if ref is None:
            monkeypatch.delenv("GLASS_AMD_PCG_NO_PREFETCH")
            ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
            monkeypatch.setenv("GLASS_AMD_PCG_NO_PREFETCH", "1")
        got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                      pinv_diagonal_blocks=True)
        for u, v in zip(ref, got):
            np.testing.assert_array_equal(u, v)


def test_resident_random_shapes_match_streamed(gpu, monkeypatch):
    """Seeded random shapes in the resident placements, whose p and r blocks
    sit in LDS padded to whole 16-byte vectors (ss=6 in blocks of 8, ss=14
    in blocks of 16) and whose dots load the chunk slots in one round trip:
    kp from 1 up to the placement's limit (ragged last chunks, 1 to 16
    waves), both preconditioners, zero and random x0, one and two rows per
    lane.  Bit for bit the streamed placement (blocks of ss, slot-by-slot
    dot), and the oracle bar on the first cases."""
    rng = np.random.default_rng(20261204)
    shapes = [(6, 170), (14, 73)]
    # the smallest systems would go to the several-per-wave placement
    monkeypatch.setenv("GLASS_AMD_PCG_MULTI", "0")
    for case in range(16):
        ss, kmax = shapes[case % 2]
        kp = int(rng.integers(1, kmax + 1))
        B = int(rng.integers(1, 70))
        rpt = "2" if case % 4 == 2 else None
        monkeypatch.delenv("GLASS_AMD_PCG_STREAMED", raising=False)
        if rpt:
            monkeypatch.setenv("GLASS_AMD_PCG_RES_RPT", rpt)
        else:
            monkeypatch.delenv("GLASS_AMD_PCG_RES_RPT", raising=False)
        assert gpu.pcg_batched_placement(ss, kp, torch.float32) == gpu.PLACEMENT_RESIDENT, (ss, kp)
        r2 = np.random.default_rng(int(rng.integers(0, 1 << 30)))
        S, D = workloads.random_spd_strips(r2, B, ss, kp, 0.2)
        P = workloads.block_tridiagonal_pinv(S, D, np.float32) if case % 3 == 1 else \
            workloads.block_jacobi_pinv(D, np.float32)
        inp = {"S": S.astype(np.float32), "Pinv": P,
               "b": r2.standard_normal((B, kp * ss)).astype(np.float32),
               "x0": (r2.standard_normal((B, kp * ss)) if case % 4 == 3
                      else np.zeros((B, kp * ss))).astype(np.float32)}
        say("resident random shape %d: ss=%d kp=%d B=%d rows/lane=%s" % (case, ss, kp, B, rpt or "1"))
        got = pcg_gpu(gpu, inp, ss, kp, 300, 1e-6, 0.0)
        monkeypatch.delenv("GLASS_AMD_PCG_RES_RPT", raising=False)
        monkeypatch.setenv("GLASS_AMD_PCG_STREAMED", "1")
        ref = pcg_gpu(gpu, inp, ss, kp, 300, 1e-6, 0.0)
        for u, v in zip(got, ref):
            np.testing.assert_array_equal(u, v)
        if case < 4:
            assert_pcg_parity(inp, ss, kp, 300, 1e-6, 0.0, got, np.float32)


@pytest.mark.parametrize("rpt", ["2", "3", "4"])
def test_pcg_resident_rows_per_lane_bit_identical(gpu, monkeypatch, rpt):
    """Resident rows at 2, 3 and 4 rows per lane (GLASS_AMD_PCG_RES_RPT; for
    the ss=6 kp=32 workload 3 rows per lane is one wave per problem) give the
    same bits as one row per lane, with and without the block-diagonal Pinv
    hint, and meet the oracle."""
    w = workloads.WORKLOADS[0]
    inp = workloads.generate(w)
    ref = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol)
    monkeypatch.setenv("GLASS_AMD_PCG_RES_RPT", rpt)
    assert gpu.pcg_batched_placement(w.ss, w.kp, torch.float32) == gpu.PLACEMENT_RESIDENT
    for pd in (False, True):
        say("pcg cfg0 resident rows/lane=%s pinv_diag=%s" % (rpt, pd))
        got = pcg_gpu(gpu, inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol,
                      pinv_block_diagonal=pd)
        for u, v in zip(ref, got):
            np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, w.ss, w.kp, w.max_iters, w.rel_tol, w.abs_tol, got, np.float32)
    if rpt == "2":
        w2 = workloads.WORKLOADS[2]
        inp2 = workloads.generate(w2, n_problems=64)
        monkeypatch.delenv("GLASS_AMD_PCG_RES_RPT")
        ref2 = pcg_gpu(gpu, inp2, w2.ss, w2.kp, w2.max_iters, w2.rel_tol, w2.abs_tol)
        monkeypatch.setenv("GLASS_AMD_PCG_RES_RPT", "2")
        say("pcg cfg2 resident rows/lane=2")
        got2 = pcg_gpu(gpu, inp2, w2.ss, w2.kp, w2.max_iters, w2.rel_tol, w2.abs_tol)
        for u, v in zip(ref2, got2):
            np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("ss,kp,B,dtype", [
    (21, 64, None, np.float32),   # the ss=21 workload, all 2048 problems
    (21, 20, 3, np.float32),      # 7 chunks: one row per lane, 7 waves
    (21, 40, 5, np.float32),      # 14 chunks: two rows per lane
    (21, 60, 4, np.float32),      # 20 chunks, the last one ragged (1260 rows)
    (21, 4, 2, np.float32),       # two chunks, the second ragged (84 rows)
    (14, 32, 40, np.float64),     # the ss=14 workload in float64
    (12, 70, 3, np.float64),      # 14 chunks, ragged, two rows per lane
])
def test_pcg_s_resident_matches_streamed(gpu, monkeypatch, ss, kp, B, dtype):
    """S-resident placement (S rows in registers, Pinv chunks loaded straight
    into the LDS stage, the last chunk of some waves pinned in the LDS left
    over): the same terms in the same order as the streamed placements and as
    the same placement without pinned chunks, so bit-identical outputs, and
    the oracle bars on every problem.  (The placement needs every problem's matrices on a 16-byte
    boundary: kp*ss a multiple of 4 in float32.)"""
    if ss == 21 and kp == 64:
        w = workloads.WORKLOADS[3]
        inp = workloads.generate(w)
        max_iters, rel, abs_tol = w.max_iters, w.rel_tol, w.abs_tol
    elif ss == 14 and kp == 32:
        w = workloads.WORKLOADS[2]
        inp = {k: v.astype(dtype) for k, v in workloads.generate(w, n_problems=B).items()}
        max_iters, rel, abs_tol = w.max_iters, w.rel_tol, w.abs_tol
    else:
        rng = np.random.default_rng(ss * 1000 + kp)
        S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.1, dtype)
        inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
               "b": rng.standard_normal((B, kp * ss)).astype(dtype),
               "x0": rng.standard_normal((B, kp * ss)).astype(dtype)}
        max_iters, rel, abs_tol = 300, (1e-8 if dtype == np.float32 else 1e-14), 0.0
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    assert gpu.pcg_batched_placement(ss, kp, tdt) == gpu.PLACEMENT_S_RESIDENT
    say("pcg ss=%d kp=%d B=%d %s S-resident" % (ss, kp, inp["b"].shape[0], np.dtype(dtype).name))
    got = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
    assert np.all(got[2] == gpu.CONVERGED)
    monkeypatch.setenv("GLASS_AMD_PCG_NO_PIN", "1")
    say("  no chunks pinned in LDS")
    unpinned = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
    monkeypatch.delenv("GLASS_AMD_PCG_NO_PIN")
    monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
    assert gpu.pcg_batched_placement(ss, kp, tdt) != gpu.PLACEMENT_S_RESIDENT
    say("  streamed reference placement")
    ref = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
    for u, v, w in zip(ref, got, unpinned):
        np.testing.assert_array_equal(u, v)
        np.testing.assert_array_equal(w, v)
    assert_pcg_parity(inp, ss, kp, max_iters, rel, abs_tol, got, dtype)


@pytest.mark.parametrize("ss,kp,B,dtype", [
    (21, 64, None, np.float32),   # the ss=21 workload, all 2048 problems
    (21, 60, 4, np.float32),      # 20 chunks, ragged last chunk
    (21, 52, 3, np.float32),      # 18 chunks on 6 waves, ragged
    (14, 32, 40, np.float64),     # the ss=14 workload in float64
    (21, 10, 3, np.float64),      # 4 chunks, one row per lane
])
def test_pcg_packed_pinv_in_lds_matches_streamed(gpu, monkeypatch, ss, kp, B, dtype):
    """Pinv's D blocks in LDS with S in registers (both matrices read once per
    solve): loaded whole when Pinv comes as packed D blocks, gathered from the
    [L|D|R] rows under the block-diagonal hint.  The same terms in the same
    order as the streamed placements of both forms and as the general
    contraction: bit-identical outputs, and the oracle bars.  (Shapes whose S
    and D rows do not fit the register-resident placement.)"""
    if (ss, kp) in ((21, 64), (14, 32)):
        w = workloads.WORKLOADS[3 if ss == 21 else 2]
        inp = {k: v.astype(dtype) for k, v in workloads.generate(w, n_problems=B).items()}
        max_iters, rel, abs_tol = w.max_iters, w.rel_tol, w.abs_tol
    else:
        rng = np.random.default_rng(ss * 1000 + kp + 7)
        S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.1, dtype)
        inp = {"S": S, "Pinv": workloads.block_jacobi_pinv(D, dtype),
               "b": rng.standard_normal((B, kp * ss)).astype(dtype),
               "x0": rng.standard_normal((B, kp * ss)).astype(dtype)}
        max_iters, rel, abs_tol = 300, (1e-8 if dtype == np.float32 else 1e-14), 0.0
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    assert gpu.pcg_batched_placement(ss, kp, tdt, pinv_diagonal_blocks=True) == \
        gpu.PLACEMENT_RESIDENT
    say("pcg ss=%d kp=%d B=%d %s packed D blocks in LDS" % (ss, kp, inp["b"].shape[0],
                                                           np.dtype(dtype).name))
    assert gpu.pcg_batched_placement(ss, kp, tdt, pinv_block_diagonal=True) == \
        gpu.PLACEMENT_RESIDENT
    got = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol, pinv_diagonal_blocks=True)
    assert np.all(got[2] == gpu.CONVERGED)
    say("  D parts gathered from [L|D|R] rows (block-diagonal hint)")
    hinted = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol, pinv_block_diagonal=True)
    general = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol)
    monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
    assert gpu.pcg_batched_placement(ss, kp, tdt, pinv_diagonal_blocks=True) != \
        gpu.PLACEMENT_RESIDENT
    say("  streamed placements, packed and hinted")
    ref = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol, pinv_diagonal_blocks=True)
    ref_h = pcg_gpu(gpu, inp, ss, kp, max_iters, rel, abs_tol, pinv_block_diagonal=True)
    for u, v, g, h, rh in zip(ref, got, general, hinted, ref_h):
        np.testing.assert_array_equal(u, v)
        np.testing.assert_array_equal(g, v)
        np.testing.assert_array_equal(h, v)
        np.testing.assert_array_equal(rh, v)
    assert_pcg_parity(inp, ss, kp, max_iters, rel, abs_tol, got, dtype)


@pytest.mark.parametrize("ss,kp,dtype,flag", [
    (21, 40, np.float32, None),           # S in registers, Pinv streamed, chunks pinned
    (21, 64, np.float32, None),
    (21, 64, np.float32, "block_diagonal"),   # D parts gathered into LDS
    (21, 64, np.float32, "diagonal_blocks"),  # packed D blocks in LDS
    (14, 32, np.float64, None),           # one row per lane, no pinned chunk
])
def test_pcg_s_resident_status_cases(gpu, monkeypatch, ss, kp, dtype, flag):
    """The S-resident placements through the status paths: breakdown on a
    negative definite system and on a NaN input, rho_init = 0, max_iters = 0
    and an exhausted max_iters, each a problem of one batch.  Statuses match
    the oracle, and every output matches the streamed placement bit for bit
    (the solve stops after a started load into the stage, or none)."""
    rng = np.random.default_rng(ss * 7 + kp)
    B = 6
    S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.2, dtype)
    P = workloads.block_jacobi_pinv(D, dtype)
    b = rng.standard_normal((B, kp * ss)).astype(dtype)
    x0 = rng.standard_normal((B, kp * ss)).astype(dtype)
    S[1] = -S[1]            # negative definite -> breakdown at the first step
    b[2] = 0.0              # with x0 = 0: rho_init == 0 -> converged, 0 iterations
    x0[2] = 0.0
    b[3, 7] = np.nan        # NaN -> breakdown, no hang
    inp = {"S": S, "Pinv": P, "b": b, "x0": x0}
    kw = {"pinv_block_diagonal": flag == "block_diagonal",
          "pinv_diagonal_blocks": flag == "diagonal_blocks"}
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    place = gpu.pcg_batched_placement(ss, kp, tdt, **kw)
    assert place == (gpu.PLACEMENT_S_RESIDENT if flag is None else gpu.PLACEMENT_RESIDENT)
    prec = "f32" if dtype == np.float32 else "f64"
    runs = {}
    for hyb in (True, False):
        if not hyb:
            monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
        for max_iters, rel, abs_tol in ((60, 1e-6, 0.0), (0, 1e-6, 0.0), (2, 0.0, 0.0),
                                        (60, 0.0, 1e30)):
            say("pcg ss=%d kp=%d %s flag=%s hybrid=%s max_iters=%d"
                % (ss, kp, np.dtype(dtype).name, flag, hyb, max_iters))
            runs[(hyb, max_iters, abs_tol)] = pcg_gpu(gpu, inp, ss, kp, max_iters, rel,
                                                      abs_tol, **kw)
    for key in [k for k in runs if k[0]]:
        for u, v in zip(runs[key], runs[(False,) + key[1:]]):
            np.testing.assert_array_equal(u, v)
    x, it, st, _ = runs[(True, 60, 0.0)]
    _, ito, sto, _ = oracle.pcg(x0, S, P, b, ss, kp, 60, 1e-6, 0.0, prec)
    np.testing.assert_array_equal(st, sto)
    assert st[1] == gpu.BREAKDOWN and it[1] == 0
    assert st[2] == gpu.CONVERGED and it[2] == 0 and np.all(x[2] == 0)
    assert st[3] == gpu.BREAKDOWN and it[3] == 0
    assert np.all(np.abs(it - ito) <= 2)
    x, it, st, _ = runs[(True, 0, 0.0)]
    assert np.all(it == 0) and st[0] == gpu.MAX_ITERS
    np.testing.assert_array_equal(x[0], x0[0])
    x, it, st, _ = runs[(True, 2, 0.0)]
    assert np.all(it[[0, 4, 5]] == 2) and np.all(st[[0, 4, 5]] == gpu.MAX_ITERS)
    x, it, st, _ = runs[(True, 60, 1e30)]
    assert np.all(it == 0) and np.all(st[[0, 2, 4, 5]] == gpu.CONVERGED)


def _shifted_copy(a, elems):
    """A device copy of array a that starts `elems` elements past a 16-byte
    boundary (the tensor is a view into a slightly larger buffer)."""
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    store = torch.zeros(t.numel() + 4, dtype=t.dtype, device="cuda")
    view = store[elems:elems + t.numel()].view(t.shape)
    view.copy_(t)
    assert view.data_ptr() % 16 == elems * t.element_size() % 16
    return view


@pytest.mark.parametrize("ss,kp,B,dtype,shift_s,shift_p,pinv", [
    (21, 64, None, np.float32, 1, 2, "tridiagonal"),   # the ss=21 workload, all problems
    (21, 64, 64, np.float32, 3, 0, "block_jacobi"),
    (21, 60, 5, np.float32, 2, 1, "tridiagonal"),      # ragged last chunk
    (21, 41, 3, np.float32, 1, 1, "tridiagonal"),      # per-problem offsets not 16-byte multiples
    (14, 32, 24, np.float64, 1, 0, "tridiagonal"),     # no spare stage bytes: streamed fallback
    (14, 32, 96, np.float32, 1, 3, "tridiagonal"),     # resident rows, element loads
])
def test_pcg_element_aligned_matrices(gpu, ss, kp, B, dtype, shift_s, shift_p, pinv):
    """S and Pinv aligned to the element size only (shifted by whole elements
    from a 16-byte boundary): the S-resident placement loads each chunk from
    the 16-byte boundary below it and reads the stage at the shift, other
    placements use element loads; the results equal the aligned call bit
    for bit and meet the oracle."""
    if B is None:
        w = replace(workloads.WORKLOADS[3], pinv=pinv)
        inp = workloads.generate(w)
    else:
        rng = np.random.default_rng(ss * 100 + kp + shift_s)
        S, D = workloads.random_spd_strips(rng, B, ss, kp, 0.1)
        P = workloads.block_tridiagonal_pinv(S, D, dtype) if pinv == "tridiagonal" else \
            workloads.block_jacobi_pinv(D, dtype)
        inp = {"S": S.astype(dtype), "Pinv": P,
               "b": rng.standard_normal((B, kp * ss)).astype(dtype),
               "x0": np.zeros((B, kp * ss), dtype)}
    B = inp["b"].shape[0]
    rel = 1e-6 if dtype == np.float32 else 1e-12
    ref = pcg_gpu(gpu, inp, ss, kp, 300, rel, 0.0)
    say("pcg ss=%d kp=%d B=%d %s, S +%d and Pinv +%d elements from 16 bytes"
        % (ss, kp, B, np.dtype(dtype).name, shift_s, shift_p))
    S_t, P_t = _shifted_copy(inp["S"], shift_s), _shifted_copy(inp["Pinv"], shift_p)
    x = torch.from_numpy(inp["x0"]).cuda().clone()
    it = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    st = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, 2), dtype=x.dtype, device="cuda")
    gpu.pcg_batched(x, S_t, P_t, torch.from_numpy(inp["b"]).cuda(), ss, kp, 300, rel, 0.0,
                    it, st, rho)
    torch.cuda.synchronize()
    got = (x.cpu().numpy(), it.cpu().numpy(), st.cpu().numpy(), rho.cpu().numpy())
    for u, v in zip(ref, got):
        np.testing.assert_array_equal(u, v)
    assert_pcg_parity(inp, ss, kp, 300, rel, 0.0, got, dtype)


def test_tuning_switches_need_the_tuning_gate(gpu):
    """The library's GLASS_AMD_* switches change a placement only in a process
    that set GLASS_AMD_TUNING=1 before the library's first call; in any other
    process the same switch is ignored (and no call reads the environment)."""
    import os
    import subprocess
    import sys
    from conftest import ROOT
    code = ("import torch, block_tridiagonal_pcg_bdmv_amd as g; g.load(); "
            "print(g.pcg_batched_placement(21, 64, torch.float32))")

    def placement(tuning):
        env = dict(os.environ)
        env["GLASS_AMD_PCG_NO_HYBRID"] = "1"
        env.pop("GLASS_AMD_TUNING", None)
        if tuning:
            env["GLASS_AMD_TUNING"] = "1"
        say("placement query in a child process, GLASS_AMD_TUNING %s" % ("set" if tuning else "unset"))
        r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                           text=True, timeout=180)
        assert r.returncode == 0, r.stderr[-2000:]
        return int(r.stdout.strip().splitlines()[-1])

    assert placement(False) == gpu.PLACEMENT_S_RESIDENT
    assert placement(True) == gpu.PLACEMENT_STREAMED_PREFETCH


def test_pinv_pass_rows_follow_the_chunk_walk(gpu, monkeypatch):
    """Pinv rows each matvec pass reads from memory.  The ss=21 kp=64
    S-resident solve: all 1344 rows at pass 0 (256 of them then stay on
    chip), after that its 17 streamed chunks less the one each of its 8 waves
    carries over in its stage, 9 chunks (576 rows).  The fp64 ss=14 solve in
    the same placement has one chunk per wave, so after pass 0 it reads
    nothing.  Resident: pass 0 only; streamed: every row every pass."""
    f32, f64 = torch.float32, torch.float64
    q = gpu.pcg_batched_pinv_pass_rows
    assert gpu.pcg_batched_placement(21, 64, f32) == gpu.PLACEMENT_S_RESIDENT
    assert (q(21, 64, f32, 0), q(21, 64, f32, 1), q(21, 64, f32, 2), q(21, 64, f32, 7)) == \
        (1344, 576, 576, 576)
    assert gpu.pcg_batched_placement(14, 32, f64) == gpu.PLACEMENT_S_RESIDENT
    assert (q(14, 32, f64, 0), q(14, 32, f64, 1), q(14, 32, f64, 2)) == (448, 0, 0)
    assert gpu.pcg_batched_placement(14, 32, f32) == gpu.PLACEMENT_RESIDENT
    assert (q(14, 32, f32, 0), q(14, 32, f32, 3)) == (448, 0)
    monkeypatch.setenv("GLASS_AMD_PCG_NO_PIN", "1")
    assert q(21, 64, f32, 0) == 1344 and q(21, 64, f32, 1) == q(21, 64, f32, 2) < 1344
    monkeypatch.setenv("GLASS_AMD_PCG_NO_HYBRID", "1")
    assert (q(21, 64, f32, 0), q(21, 64, f32, 1)) == (1344, 1344)
