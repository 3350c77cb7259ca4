"""GPU parity of glass_bdmv_batched against the CPU oracle (float64 reference),
bar: |err| <= 1e-5 * the row's absolute sum.  Every call goes through the C ABI."""

import os

import numpy as np
import pytest
import torch

import workloads
from gpu_common import assert_bdmv_close, bdmv_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def random_case(seed, B, ss, kp, dtype, garbage=True):
    rng = np.random.default_rng(seed)
    S = rng.uniform(-1, 1, (B, kp, ss, 3 * ss))
    if not garbage:
        S[:, 0, :, :ss] = 0
        S[:, -1, :, 2 * ss:] = 0
    v = np.zeros((B, (kp + 2) * ss))
    v[:, ss:-ss] = rng.standard_normal((B, kp * ss))
    return S.astype(dtype), v.astype(dtype)


def test_bdmv_workload_shape_several_tiles_ragged(gpu):
    """ss=14, kp=64: 896 rows per problem = 3 full 256-row tiles + a half tile."""
    w = workloads.WORKLOADS[1]
    inp = workloads.generate(w, n_problems=37)
    say("bdmv ss=14 kp=64 B=37")
    y = bdmv_gpu(gpu, inp["S"], inp["v"], w.ss, w.kp)
    assert_bdmv_close(y, inp["S"], inp["v"], w.ss, w.kp)
    assert np.all(np.isnan(y[:, :w.ss])) and np.all(np.isnan(y[:, -w.ss:])), "pads written"


def test_bdmv_full_workload_all_problems(gpu):
    """The full 8192-problem fp32 workload, every row checked."""
    w = workloads.WORKLOADS[1]
    inp = workloads.generate(w)
    say("bdmv full ss=14 kp=64 B=8192")
    y = bdmv_gpu(gpu, inp["S"], inp["v"], w.ss, w.kp)
    assert_bdmv_close(y, inp["S"], inp["v"], w.ss, w.kp)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("ss,kp,B", [(1, 1, 3), (1, 300, 2), (2, 3, 5), (5, 7, 4),
                                     (6, 32, 9), (12, 20, 3), (14, 1, 6), (21, 64, 2),
                                     (33, 5, 2), (64, 3, 2)])
def test_bdmv_edge_shapes(gpu, ss, kp, B, dtype):
    S, v = random_case(ss * 1000 + kp, B, ss, kp, dtype)
    say("bdmv ss=%d kp=%d B=%d %s" % (ss, kp, B, np.dtype(dtype).name))
    y = bdmv_gpu(gpu, S, v, ss, kp)
    assert_bdmv_close(y, S, v, ss, kp)
    assert np.all(np.isnan(y[:, :ss])) and np.all(np.isnan(y[:, -ss:]))


def test_bdmv_zero_pad_invariance(gpu):
    """Finite garbage in the off-matrix blocks L_0 and R_{kp-1} multiplies the
    zero pads: the result is bit-identical to zero blocks."""
    S, v = random_case(5, 6, 14, 9, np.float32, garbage=True)
    S0 = S.copy()
    S0[:, 0, :, :14] = 0
    S0[:, -1, :, 28:] = 0
    say("bdmv pad invariance")
    np.testing.assert_array_equal(bdmv_gpu(gpu, S, v, 14, 9), bdmv_gpu(gpu, S0, v, 14, 9))


def test_bdmv_thread_count_invariance(gpu, monkeypatch):
    """One thread owns one row and sums it in a fixed order, so the output is
    bit-identical for every workgroup size."""
    S, v = random_case(9, 5, 14, 40, np.float32)
    outs = []
    for nt in (64, 128, 192, 256):
        monkeypatch.setenv("GLASS_AMD_BDMV_THREADS", str(nt))
        say("bdmv threads=%d" % nt)
        outs.append(bdmv_gpu(gpu, S, v, 14, 40))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_bdmv_unaligned_base_uses_scalar_path(gpu):
    """A base pointer that is element- but not 16-byte-aligned must give the
    same bits as the aligned call."""
    S, v = random_case(13, 3, 6, 10, np.float32)
    aligned = bdmv_gpu(gpu, S, v, 6, 10)
    big = torch.zeros(S.size + 1, dtype=torch.float32, device="cuda")
    big[1:] = to_dev(S).reshape(-1)
    Sv = big[1:]
    assert Sv.data_ptr() % 16 != 0
    vt = to_dev(v)
    y = torch.full_like(vt, float("nan"))
    say("bdmv unaligned S")
    gpu.bdmv_batched(y, Sv, vt, 6, 10)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), aligned)


def test_bdmv_zero_problems_is_a_no_op(gpu):
    S = torch.zeros(0, dtype=torch.float32, device="cuda")
    y = torch.zeros(0, dtype=torch.float32, device="cuda")
    gpu.bdmv_batched(y, S, y, 14, 64)
    torch.cuda.synchronize()


def test_bdmv_rejects_wrong_sizes_before_launch(gpu):
    S, v = random_case(1, 2, 4, 5, np.float32)
    St, vt = to_dev(S), to_dev(v)
    with pytest.raises(ValueError):
        gpu.bdmv_batched(torch.zeros(5, device="cuda"), St, vt, 4, 5)
    with pytest.raises(TypeError):
        gpu.bdmv_batched(torch.zeros_like(vt, dtype=torch.float64), St, vt, 4, 5)
