"""Seeded synthetic inputs for the block-tridiagonal bdmv / PCG workloads.

This module builds inputs only.  It holds none of the method's arithmetic (no
matvec, no dot, no CG step) and is shared by the tests, the smoke check and the
benchmark; both the CPU oracle and the HIP library consume what it returns.

Layouts (GLASS user guide, page "Block-tridiagonal Solves"):
* S and Pinv: ``[n_problems, kp, ss, 3*ss]`` -- kp row-major strips holding
  [L_br | D_br | R_br] (section "The [L|D|R] block-tridiagonal layout");
* bdmv vectors: ``[n_problems, (kp+2)*ss]`` with zero pad blocks at both ends
  (section "The padded vector layout");
* PCG x and b: unpadded ``[n_problems, kp*ss]`` (the C ABI's reading: the page
  keeps padded vectors as the solver's internal scratch).

Recipe, per problem and in this draw order, from one
``numpy.random.Generator(PCG64(seed))``:
1. ``R_raw``: (kp-1, ss, ss) uniform [0,1); R_br = R_raw[br] - 0.5.
2. ``U_raw``: (kp, ss, ss) uniform [0,1); the strict upper triangle of
   U_raw[br] - 0.5 gives D_br's off-diagonal entries, mirrored to keep D_br
   symmetric (the lower triangle and diagonal of U_raw are drawn and unused).
3. the right-hand side b (or the bdmv input vector): kp*ss standard normals.
Then L_{br+1} = R_br^T, L_0 = 0, R_{kp-1} = 0, and each diagonal entry of
D_br is the absolute sum of the rest of its full matrix row (L, D and R
blocks) plus ``margin``.  By Gershgorin every eigenvalue is at least
``margin``, so S is symmetric positive definite and diagonally dominant.
Pinv is block-Jacobi: its D part is inv(D_br) computed in float64 and
symmetrised, its L/R parts are zero.  x0 = 0.  Everything is formed in float64
and rounded once to the workload dtype.

Preconditioner option ``pinv="tridiagonal"`` (the same page lets Pinv be any
block-tridiagonal matrix in [L|D|R] form; this choice is ours): the
first-order Neumann approximation of S^-1 about its block diagonal,
    Pinv = D^-1 - D^-1 E D^-1,   E = the L and R blocks of S,
so Pinv's D blocks are inv(D_br), its R blocks -inv(D_br) R_br inv(D_br+1) and
its L blocks the transposes of the R blocks of the row above.  With
F = D^-1/2 E D^-1/2, Pinv = D^-1/2 (I - F) D^-1/2.  F is block-tridiagonal
with zero diagonal blocks (2-cyclic), so its spectrum is symmetric about 0;
S = D^1/2 (I + F) D^1/2 SPD means every eigenvalue of F exceeds -1, hence
all lie in (-1, 1) and Pinv is SPD too.  Pinv S is similar to I - F^2.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "pcg", "bdmv" or "grid"
    dtype: type
    ss: int              # state_size
    kp: int              # knot_points
    n_problems: int
    margin: float
    rel_tol: float = 0.0
    abs_tol: float = 0.0
    max_iters: int = 0
    seed: int = 0
    pinv: str = "block_jacobi"   # or "tridiagonal" (see the module docstring)

    @property
    def n(self) -> int:
        return self.kp * self.ss

    def with_problems(self, n_problems: int) -> "Workload":
        return replace(self, n_problems=int(n_problems))


# The five workloads of the hot path.  Seed = 1000 + index.
WORKLOADS = {
    0: Workload("pcg_ss6_kp32_b64_f32", "pcg", np.float32, 6, 32, 64, 1.0,
                rel_tol=1e-6, abs_tol=0.0, max_iters=200, seed=1000),
    1: Workload("bdmv_ss14_kp64_b8192_f32", "bdmv", np.float32, 14, 64, 8192,
                1.0, seed=1001),
    2: Workload("pcg_ss14_kp32_b4096_f32", "pcg", np.float32, 14, 32, 4096,
                0.2, rel_tol=1e-6, abs_tol=0.0, max_iters=200, seed=1002),
    3: Workload("pcg_ss21_kp64_b2048_f32", "pcg", np.float32, 21, 64, 2048,
                0.1, rel_tol=1e-6, abs_tol=0.0, max_iters=500, seed=1003),
    4: Workload("grid_pcg_ss12_kp8192_f64", "grid", np.float64, 12, 8192, 1,
                0.05, rel_tol=1e-10, abs_tol=0.0, max_iters=2000, seed=1004),
}


def _assemble(R: np.ndarray, U: np.ndarray, ss: int, kp: int, margin: float):
    """Float64 strips [B, kp, ss, 3ss] and D blocks [B, kp, ss, ss]."""
    B = U.shape[0]
    S = np.zeros((B, kp, ss, 3 * ss), dtype=np.float64)
    iu = np.triu_indices(ss, 1)
    D = np.zeros((B, kp, ss, ss), dtype=np.float64)
    D[:, :, iu[0], iu[1]] = U[:, :, iu[0], iu[1]]
    D = D + np.swapaxes(D, -1, -2)
    if kp > 1:
        S[:, :-1, :, 2 * ss:] = R                      # R_br, br < kp-1
        S[:, 1:, :, :ss] = np.swapaxes(R, -1, -2)       # L_{br+1} = R_br^T
    offsum = np.abs(S[:, :, :, :ss]).sum(-1) + np.abs(S[:, :, :, 2 * ss:]).sum(-1) \
        + np.abs(D).sum(-1)
    di = np.arange(ss)
    D[:, :, di, di] = offsum + margin
    S[:, :, :, ss:2 * ss] = D
    return S, D


def generate(w: Workload, n_problems: int | None = None, with_pinv: bool | None = None,
             chunk: int = 512):
    """Build the inputs of workload ``w`` (optionally only its first
    ``n_problems`` problems -- the draws are per problem, so a prefix of the
    batch is identical to the same problems of the full batch).

    Returns a dict with ``S``, ``Pinv`` (PCG kinds), ``b`` and ``x0`` (PCG
    kinds) or ``v`` (bdmv kind), all C-contiguous numpy arrays of ``w.dtype``.
    """
    B = w.n_problems if n_problems is None else int(n_problems)
    ss, kp = w.ss, w.kp
    if with_pinv is None:
        with_pinv = w.kind != "bdmv"
    rng = np.random.Generator(np.random.PCG64(w.seed))
    S_out = np.empty((B, kp, ss, 3 * ss), dtype=w.dtype)
    P_out = np.empty((B, kp, ss, 3 * ss), dtype=w.dtype) if with_pinv else None
    if w.kind == "bdmv":
        vec_out = np.zeros((B, (kp + 2) * ss), dtype=w.dtype)
    else:
        vec_out = np.empty((B, kp * ss), dtype=w.dtype)
    for lo in range(0, B, chunk):
        hi = min(B, lo + chunk)
        m = hi - lo
        R = np.empty((m, max(kp - 1, 0), ss, ss), dtype=np.float64)
        U = np.empty((m, kp, ss, ss), dtype=np.float64)
        g = np.empty((m, kp * ss), dtype=np.float64)
        for q in range(m):
            rng.random(out=R[q])
            rng.random(out=U[q])
            rng.standard_normal(out=g[q])
        R -= 0.5
        U -= 0.5
        S, D = _assemble(R, U, ss, kp, w.margin)
        S_out[lo:hi] = S
        if with_pinv:
            if w.pinv == "tridiagonal":
                P_out[lo:hi] = _tridiagonal_pinv64(S, D)
            elif w.pinv == "block_jacobi":
                inv = np.linalg.inv(D)
                inv = 0.5 * (inv + np.swapaxes(inv, -1, -2))
                P = np.zeros_like(S)
                P[:, :, :, ss:2 * ss] = inv
                P_out[lo:hi] = P
            else:
                raise ValueError("unknown preconditioner %r" % (w.pinv,))
        if w.kind == "bdmv":
            vec_out[lo:hi, ss:(kp + 1) * ss] = g
        else:
            vec_out[lo:hi] = g
    out = {"S": S_out}
    if with_pinv:
        out["Pinv"] = P_out
    if w.kind == "bdmv":
        out["v"] = vec_out
    else:
        out["b"] = vec_out
        out["x0"] = np.zeros((B, kp * ss), dtype=w.dtype)
    return out


def identity_pinv(B: int, ss: int, kp: int, dtype=np.float64) -> np.ndarray:
    """Pinv = I in strip form (D blocks identity, L/R zero)."""
    P = np.zeros((B, kp, ss, 3 * ss), dtype=dtype)
    P[:, :, np.arange(ss), ss + np.arange(ss)] = 1.0
    return P


def random_spd_strips(rng: np.random.Generator, B: int, ss: int, kp: int,
                      margin: float, dtype=np.float64, offdiag: bool = True):
    """Same recipe as ``generate`` from a caller-owned generator (test sizes);
    ``offdiag=False`` gives a block-diagonal S (all R, L zero).
    Returns (S, D) in float64 rounded to ``dtype``."""
    R = rng.random((B, max(kp - 1, 0), ss, ss)) - 0.5
    if not offdiag:
        R[:] = 0.0
    U = rng.random((B, kp, ss, ss)) - 0.5
    S, D = _assemble(R, U, ss, kp, margin)
    return S.astype(dtype), D


def block_jacobi_pinv(D: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Block-Jacobi preconditioner strips from float64 D blocks [B, kp, ss, ss]."""
    B, kp, ss, _ = D.shape
    inv = np.linalg.inv(D)
    inv = 0.5 * (inv + np.swapaxes(inv, -1, -2))
    P = np.zeros((B, kp, ss, 3 * ss), dtype=np.float64)
    P[:, :, :, ss:2 * ss] = inv
    return P.astype(dtype)


def _tridiagonal_pinv64(S: np.ndarray, D: np.ndarray) -> np.ndarray:
    """Float64 strips of Pinv = D^-1 - D^-1 E D^-1 (module docstring) for
    float64 strips S [B, kp, ss, 3ss] with D blocks D [B, kp, ss, ss]."""
    B, kp, ss, _ = D.shape
    inv = np.linalg.inv(D)
    inv = 0.5 * (inv + np.swapaxes(inv, -1, -2))
    P = np.zeros((B, kp, ss, 3 * ss), dtype=np.float64)
    P[:, :, :, ss:2 * ss] = inv
    if kp > 1:
        R = S[:, :-1, :, 2 * ss:]
        PR = -np.matmul(np.matmul(inv[:, :-1], R), inv[:, 1:])
        P[:, :-1, :, 2 * ss:] = PR
        P[:, 1:, :, :ss] = np.swapaxes(PR, -1, -2)
    return P


def block_tridiagonal_pinv(S: np.ndarray, D: np.ndarray, dtype=np.float64) -> np.ndarray:
    """The SPD block-tridiagonal preconditioner of ``pinv="tridiagonal"``
    (non-zero L and R blocks) for strips S built by ``random_spd_strips`` /
    ``generate`` (symmetric, L_{br+1} = R_br^T) and their float64 D blocks."""
    return _tridiagonal_pinv64(np.asarray(S, np.float64), np.asarray(D, np.float64)).astype(dtype)


def laplacian_coupled_strips(S: np.ndarray, scale: float) -> np.ndarray:
    """A stiffer SPD system for long solves: scale * S plus the block 1-D
    Laplacian tridiag(-I, 2I, -I) (positive semidefinite, eigenvalues
    2 - 2 cos(k pi / (kp+1)) > 0), so the sum stays symmetric positive
    definite while its condition number grows as scale shrinks.  S: strips
    [B, kp, ss, 3ss] of a symmetric S; returns float64 strips."""
    S = scale * np.asarray(S, np.float64)
    ss = S.shape[2]
    eye = np.eye(ss)
    S[:, :, :, ss:2 * ss] += 2.0 * eye
    if S.shape[1] > 1:
        S[:, :-1, :, 2 * ss:] -= eye
        S[:, 1:, :, :ss] -= eye
    return S
