"""CPU oracle for the batched block-tridiagonal bdmv and PCG.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product library
(the HIP kernels and their C ABI) never calls it, and it shares no code with
them: the arithmetic lives in ``oracle.cpp`` (plain sequential C++, built with
g++ and ``-ffp-contract=off``); this module only builds it and marshals numpy
arrays through ctypes.

Functions and what they follow (GLASS user guide, page "Block-tridiagonal
Solves"):

* ``bdmv`` -- sections "The [L|D|R] block-tridiagonal layout" and "The padded
  vector layout": y[(br+1)*ss + i] = sum_c S[br][i][c] * v[br*ss + c].
* ``pcg`` -- section "Solve -- glass::pcg": preconditioned CG on S x = b with
  a block-tridiagonal Pinv, stopping when |r^T z| < abs_tol + rel_tol*|rho_init|.
* ``dense_expand`` -- the n x n matrix the strips stand for (same layout
  section); used to pin ``bdmv`` against a plain dense product.
* ``cholesky_solve`` -- a dense SPD solve, used to pin ``pcg`` on tiny systems.
* ``bdsv`` -- the direct solve of the same page's opening paragraph
  (glass::bdsv), whose steps the page does not give: block elimination
  without pivoting across block-rows (block Thomas; Golub and Van Loan,
  "Matrix Computations", section 4.5.1), each pivot block factored by
  Cholesky.

Pins: every function is checked in ``tests/test_oracle.py`` against something
other than itself (hand-derived fixtures under ``tests/golden/``, a dense
product built from the blocks, numpy's LU solve, the finite-termination
theorem of CG, invariants).  No function here is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

CONVERGED, MAX_ITERS, BREAKDOWN = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile ``oracle.cpp`` into ``liboracle.so`` with g++ (no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c++17",
           "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I, LL, D = ctypes.c_int, ctypes.c_longlong, ctypes.c_double
            for name in ("oracle_bdmv_f64", "oracle_bdmv_f32"):
                f = getattr(lib, name)
                f.argtypes = [P, P, P, I, I, LL, I]
                f.restype = None
            for name in ("oracle_pcg_f64", "oracle_pcg_f32"):
                f = getattr(lib, name)
                f.argtypes = [P, P, P, P, I, I, LL, I, D, D, P, P, P, I]
                f.restype = None
            for name in ("oracle_bdsv_f64", "oracle_bdsv_f32"):
                f = getattr(lib, name)
                f.argtypes = [P, P, P, I, I, LL, P, I]
                f.restype = None
            lib.oracle_dense_expand.argtypes = [P, P, I, I]
            lib.oracle_dense_expand.restype = None
            lib.oracle_cholesky_solve.argtypes = [P, P, P, I]
            lib.oracle_cholesky_solve.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def bdmv(S, v, ss: int, kp: int, precision: str = "f64", nthreads: int = 1,
         y=None) -> np.ndarray:
    """Batched y = A_bd v.

    S: [B, kp*ss*3*ss] (any shape with that many elements per problem);
    v: [B, (kp+2)*ss] padded.  ``precision`` "f64" converts the inputs to
    float64 exactly and sums in float64 (the parity reference); "f32" sums in
    float32.  Only the interiors of y are written; y defaults to zeros.
    """
    dt = np.float64 if precision == "f64" else np.float32
    vec = (kp + 2) * ss
    v = _c(v, dt).reshape(-1, vec)
    B = v.shape[0]
    S = _c(S, dt).reshape(B, -1)
    assert S.shape[1] == kp * ss * 3 * ss, "S has the wrong per-problem size"
    if y is None:
        y = np.zeros((B, vec), dtype=dt)
    else:
        y = _c(y, dt).reshape(B, vec).copy()
    fn = _load().oracle_bdmv_f64 if dt == np.float64 else _load().oracle_bdmv_f32
    fn(_ptr(y), _ptr(S), _ptr(v), ss, kp, B, nthreads)
    return y


def pcg(x0, S, Pinv, b, ss: int, kp: int, max_iters: int, rel_tol: float,
        abs_tol: float, precision: str = "f64", nthreads: int = 1):
    """Batched PCG.  Returns (x, iters, status, rho) with rho[:, 0] the signed
    initial r^T z and rho[:, 1] the last r^T z computed."""
    dt = np.float64 if precision == "f64" else np.float32
    n = kp * ss
    b = _c(b, dt).reshape(-1, n)
    B = b.shape[0]
    x = _c(x0, dt).reshape(B, n).copy()
    S = _c(S, dt).reshape(B, -1)
    Pinv = _c(Pinv, dt).reshape(B, -1)
    assert S.shape[1] == n * 3 * ss and Pinv.shape[1] == n * 3 * ss
    iters = np.zeros(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    rho = np.zeros((B, 2), dtype=np.float64)
    fn = _load().oracle_pcg_f64 if dt == np.float64 else _load().oracle_pcg_f32
    fn(_ptr(x), _ptr(S), _ptr(Pinv), _ptr(b), ss, kp, B, int(max_iters),
       float(rel_tol), float(abs_tol), _ptr(iters), _ptr(status), _ptr(rho),
       nthreads)
    return x, iters, status, rho


def bdsv(S, b, ss: int, kp: int, precision: str = "f64", nthreads: int = 1, x=None):
    """Batched direct solve S x = b.  Returns (x, status): status 0, or 1 when
    a pivot block is not numerically SPD (that problem's x is left as given,
    zeros by default)."""
    dt = np.float64 if precision == "f64" else np.float32
    n = kp * ss
    b = _c(b, dt).reshape(-1, n)
    B = b.shape[0]
    S = _c(S, dt).reshape(B, -1)
    assert S.shape[1] == n * 3 * ss, "S has the wrong per-problem size"
    x = np.zeros((B, n), dtype=dt) if x is None else _c(x, dt).reshape(B, n).copy()
    status = np.zeros(B, dtype=np.int32)
    fn = _load().oracle_bdsv_f64 if dt == np.float64 else _load().oracle_bdsv_f32
    fn(_ptr(x), _ptr(S), _ptr(b), ss, kp, B, _ptr(status), nthreads)
    return x, status


def dense_expand(S, ss: int, kp: int) -> np.ndarray:
    """One problem's strips as a dense (kp*ss) x (kp*ss) float64 matrix."""
    S = _c(S, np.float64).reshape(-1)
    assert S.size == kp * ss * 3 * ss
    n = kp * ss
    A = np.empty((n, n), dtype=np.float64)
    _load().oracle_dense_expand(_ptr(A), _ptr(S), ss, kp)
    return A


def cholesky_solve(A, b) -> np.ndarray:
    """Dense SPD solve by Cholesky; raises ValueError if A is not SPD."""
    A = _c(A, np.float64)
    n = A.shape[0]
    b = _c(b, np.float64).reshape(n)
    x = np.empty(n, dtype=np.float64)
    if _load().oracle_cholesky_solve(_ptr(x), _ptr(A), _ptr(b), n) != 0:
        raise ValueError("matrix is not numerically SPD")
    return x
