// CPU oracle for the batched block-tridiagonal matvec (bdmv) and the
// block-tridiagonal-preconditioned conjugate-gradient solve (pcg).
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
// or calls this file.  Only the test suite, the smoke check and the CPU
// baseline leg of the benchmark load it.  It shares no code, header, table or
// helper with the HIP kernels.
//
// Everything here is written to be checked by eye against the definitions on
// the GLASS user-guide page "Block-tridiagonal Solves":
//   * section "The [L|D|R] block-tridiagonal layout": knot_points row-major
//     strips of state_size x 3*state_size, block-row br holding [L_br|D_br|R_br];
//   * section "The padded vector layout": vectors of (knot_points+2)*state_size
//     with one zero pad block at each end; block-row br reads the window
//     v[br*ss, br*ss+3*ss) and writes y[(br+1)*ss + row];
//   * section "Solve -- glass::pcg": PCG on S x = b with preconditioner Pinv
//     (both in [L|D|R] form); convergence on the preconditioned residual
//     rho = r^T z, stop when |rho| < abs_tol + rel_tol*|rho_init|; x is the
//     initial guess on entry and the solution on exit; iters is returned.
// The PCG steps themselves are not printed on the page; the oracle follows the
// standard preconditioned CG (Hestenes and Stiefel 1952; Saad, "Iterative
// Methods for Sparse Linear Systems", Algorithm 9.1), whose initialisation
// z = p = Pinv*r the page names in section "Matvec -- glass::bdmv".
// The page's opening paragraph also names glass::bdsv, a direct solve of the
// same block-tridiagonal SPD systems, without giving its steps; the oracle
// follows block Gaussian elimination without pivoting across block-rows (the
// block Thomas algorithm; Golub and Van Loan, "Matrix Computations", section
// 4.5.1 on block tridiagonal systems), each pivot block factored by Cholesky.
//
// No blocking, fusion or reordering: every sum runs sequentially in index
// order.  Build with -ffp-contract=off so a*b+c is never fused.

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// bdmv: y = A_bd * v on one problem.  Page "Block-tridiagonal Solves",
// sections "The [L|D|R] block-tridiagonal layout" and "The padded vector
// layout".  Only the interior of y is written; its pad blocks are untouched.
// ---------------------------------------------------------------------------
template <typename T>
void bdmv_one(T* y, const T* S, const T* v, int ss, int kp) {
  const int width = 3 * ss;  // columns of one strip row: L | D | R
  for (int br = 0; br < kp; ++br) {
    const T* strip = S + (size_t)br * width * ss;  // block-row br
    const T* window = v + (size_t)br * ss;         // previous | current | next
    for (int row = 0; row < ss; ++row) {
      const T* srow = strip + (size_t)row * width;
      T acc = T(0);
      for (int c = 0; c < width; ++c) acc = acc + srow[c] * window[c];
      y[(size_t)(br + 1) * ss + row] = acc;
    }
  }
}

// Dot product over the interior of two padded vectors, in index order.
template <typename T>
T dot_interior(const T* a, const T* b, int ss, int kp) {
  T acc = T(0);
  const size_t lo = (size_t)ss, hi = (size_t)(kp + 1) * ss;
  for (size_t i = lo; i < hi; ++i) acc = acc + a[i] * b[i];
  return acc;
}

enum { PCG_CONVERGED = 0, PCG_MAX_ITERS = 1, PCG_BREAKDOWN = 2 };

struct PcgOut {
  int iters;
  int status;
  double rho_init;
  double rho_final;
};

// ---------------------------------------------------------------------------
// pcg on one problem, in precision T.  x and b are unpadded (kp*ss); the five
// work vectors (x, r, z, p, S*p) are padded as on the page so the bdmv above
// needs no edge cases.
//
// Control flow (the reading of the page's stopping rule):
//   r = b - S x;  z = Pinv r;  p = z;  rho = r^T z;  rho_init = |rho|
//   thresh = abs_tol + rel_tol * rho_init            (computed in T)
//   if rho_init == 0 or rho_init < thresh: converged, 0 iterations
//   for k = 0 .. max_iters-1:
//     Sp = S p;  pSp = p^T Sp
//     if not (pSp > 0) or pSp is not finite: breakdown (x keeps last update)
//     alpha = rho / pSp;  x += alpha p;  r -= alpha Sp;  iters = k+1
//     z = Pinv r;  rho' = r^T z
//     if |rho'| < thresh: converged
//     beta = rho' / rho;  p = z + beta p;  rho = rho'
//   if the loop runs out: max_iters
// ---------------------------------------------------------------------------
template <typename T>
PcgOut pcg_one(T* x, const T* S, const T* Pinv, const T* b, int ss, int kp,
               int max_iters, T rel_tol, T abs_tol) {
  const int n = kp * ss;
  const size_t padded = (size_t)(kp + 2) * ss;
  std::vector<T> xv(padded, T(0)), r(padded, T(0)), z(padded, T(0)),
      p(padded, T(0)), Sp(padded, T(0));
  for (int i = 0; i < n; ++i) xv[ss + i] = x[i];

  // r = b - S x
  bdmv_one(Sp.data(), S, xv.data(), ss, kp);
  for (int i = 0; i < n; ++i) r[ss + i] = b[i] - Sp[ss + i];
  // z = p = Pinv r
  bdmv_one(z.data(), Pinv, r.data(), ss, kp);
  for (int i = 0; i < n; ++i) p[ss + i] = z[ss + i];
  T rho = dot_interior(r.data(), z.data(), ss, kp);
  const T rho_init = std::fabs(rho);
  const T thresh = abs_tol + rel_tol * rho_init;

  PcgOut out{0, PCG_MAX_ITERS, (double)rho, (double)rho};
  if (rho_init == T(0) || rho_init < thresh) {
    out.status = PCG_CONVERGED;
    return out;  // x unchanged
  }
  for (int k = 0; k < max_iters; ++k) {
    bdmv_one(Sp.data(), S, p.data(), ss, kp);
    const T pSp = dot_interior(p.data(), Sp.data(), ss, kp);
    if (!(pSp > T(0)) || !std::isfinite(pSp)) {
      out.status = PCG_BREAKDOWN;
      break;
    }
    const T alpha = rho / pSp;
    for (int i = 0; i < n; ++i) {
      xv[ss + i] = xv[ss + i] + alpha * p[ss + i];
      r[ss + i] = r[ss + i] - alpha * Sp[ss + i];
    }
    out.iters = k + 1;
    bdmv_one(z.data(), Pinv, r.data(), ss, kp);
    const T rho_new = dot_interior(r.data(), z.data(), ss, kp);
    out.rho_final = (double)rho_new;
    if (std::fabs(rho_new) < thresh) {
      out.status = PCG_CONVERGED;
      break;
    }
    const T beta = rho_new / rho;
    for (int i = 0; i < n; ++i) p[ss + i] = z[ss + i] + beta * p[ss + i];
    rho = rho_new;
  }
  for (int i = 0; i < n; ++i) x[i] = xv[ss + i];
  return out;
}

// ---------------------------------------------------------------------------
// Small dense helpers for bdsv (row-major m x m blocks).
// ---------------------------------------------------------------------------

// In-place Cholesky M = C C^T (Cholesky-Banachiewicz, lower triangle of M
// receives C; the strict upper triangle is left alone).  Returns false if a
// pivot is not positive (M not numerically SPD).
template <typename T>
bool chol_inplace(T* M, int m) {
  for (int i = 0; i < m; ++i) {
    for (int j = 0; j <= i; ++j) {
      T s = M[i * m + j];
      for (int k = 0; k < j; ++k) s = s - M[i * m + k] * M[j * m + k];
      if (i == j) {
        if (!(s > T(0))) return false;
        M[i * m + i] = std::sqrt(s);
      } else {
        M[i * m + j] = s / M[j * m + j];
      }
    }
  }
  return true;
}

// X := (C C^T)^{-1} X for an m x ncol block X (row stride ncol), C from
// chol_inplace: forward substitution with C, then back substitution with C^T,
// column by column.
template <typename T>
void chol_solve_cols(const T* C, int m, T* X, int ncol) {
  for (int j = 0; j < ncol; ++j) {
    for (int i = 0; i < m; ++i) {  // C y = x
      T s = X[i * ncol + j];
      for (int k = 0; k < i; ++k) s = s - C[i * m + k] * X[k * ncol + j];
      X[i * ncol + j] = s / C[i * m + i];
    }
    for (int i = m - 1; i >= 0; --i) {  // C^T x = y
      T s = X[i * ncol + j];
      for (int k = i + 1; k < m; ++k) s = s - C[k * m + i] * X[k * ncol + j];
      X[i * ncol + j] = s / C[i * m + i];
    }
  }
}

// ---------------------------------------------------------------------------
// bdsv on one problem: S x = b by block elimination (block Thomas), in
// precision T.  With block-row br holding [L_br | D_br | R_br]:
//   M_0 = D_0,                u_0 = M_0^{-1} b_0
//   G_{br-1} = M_{br-1}^{-1} R_{br-1}
//   M_br = D_br - L_br G_{br-1},   u_br = M_br^{-1} (b_br - L_br u_{br-1})
//   x_{kp-1} = u_{kp-1},   x_br = u_br - G_br x_{br+1}
// Every M_br (a Schur complement of the SPD matrix) is factored by Cholesky.
// Returns 0, or 1 if some M_br is not numerically SPD (x is then unchanged).
// ---------------------------------------------------------------------------
template <typename T>
int bdsv_one(T* x, const T* S, const T* b, int ss, int kp) {
  const int width = 3 * ss;
  auto blk = [&](int br, int which, int i, int j) {  // which: 0 L, 1 D, 2 R
    return S[((size_t)br * ss + i) * width + which * ss + j];
  };
  // G and u of every block-row, stored side by side: [G_br | u_br], ss x (ss+1)
  const int nc = ss + 1;
  std::vector<T> GU((size_t)kp * ss * nc, T(0));
  std::vector<T> M((size_t)ss * ss);
  for (int br = 0; br < kp; ++br) {
    T* gu = GU.data() + (size_t)br * ss * nc;
    // M_br = D_br - L_br G_{br-1};  rhs = b_br - L_br u_{br-1}
    for (int i = 0; i < ss; ++i) {
      for (int j = 0; j < ss; ++j) M[i * ss + j] = blk(br, 1, i, j);
      gu[i * nc + ss] = b[(size_t)br * ss + i];
    }
    if (br > 0) {
      const T* prev = GU.data() + (size_t)(br - 1) * ss * nc;
      for (int i = 0; i < ss; ++i) {
        for (int j = 0; j < nc; ++j) {
          T s = T(0);
          for (int k = 0; k < ss; ++k) s = s + blk(br, 0, i, k) * prev[k * nc + j];
          if (j < ss) M[i * ss + j] = M[i * ss + j] - s;
          else gu[i * nc + ss] = gu[i * nc + ss] - s;
        }
      }
    }
    if (!chol_inplace(M.data(), ss)) return 1;
    // [G_br | u_br] = M_br^{-1} [R_br | rhs]   (no R for the last block-row)
    for (int i = 0; i < ss; ++i)
      for (int j = 0; j < ss; ++j) gu[i * nc + j] = br + 1 < kp ? blk(br, 2, i, j) : T(0);
    chol_solve_cols(M.data(), ss, gu, nc);
  }
  // Back substitution, from the last block-row up.
  std::vector<T> xv((size_t)kp * ss);
  for (int br = kp - 1; br >= 0; --br) {
    const T* gu = GU.data() + (size_t)br * ss * nc;
    for (int i = 0; i < ss; ++i) {
      T s = gu[i * nc + ss];
      if (br + 1 < kp)
        for (int k = 0; k < ss; ++k) s = s - gu[i * nc + k] * xv[(size_t)(br + 1) * ss + k];
      xv[(size_t)br * ss + i] = s;
    }
  }
  for (size_t i = 0; i < xv.size(); ++i) x[i] = xv[i];
  return 0;
}

// Run f(lo, hi) over [0, count) split into contiguous ranges on nthreads.
template <typename F>
void parallel_ranges(long long count, int nthreads, F f) {
  if (nthreads <= 1 || count <= 1) {
    f(0LL, count);
    return;
  }
  if ((long long)nthreads > count) nthreads = (int)count;
  std::vector<std::thread> pool;
  pool.reserve(nthreads);
  for (int t = 0; t < nthreads; ++t) {
    const long long lo = count * t / nthreads, hi = count * (t + 1) / nthreads;
    pool.emplace_back([=] { f(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

template <typename T>
void bdmv_batched(T* y, const T* S, const T* v, int ss, int kp,
                  long long n_problems, int nthreads) {
  const size_t strip = (size_t)kp * ss * 3 * ss, vec = (size_t)(kp + 2) * ss;
  parallel_ranges(n_problems, nthreads, [=](long long lo, long long hi) {
    for (long long q = lo; q < hi; ++q)
      bdmv_one(y + q * vec, S + q * strip, v + q * vec, ss, kp);
  });
}

template <typename T>
void pcg_batched(T* x, const T* S, const T* Pinv, const T* b, int ss, int kp,
                 long long n_problems, int max_iters, double rel_tol,
                 double abs_tol, int* iters_out, int* status_out,
                 double* rho_out, int nthreads) {
  const size_t strip = (size_t)kp * ss * 3 * ss, n = (size_t)kp * ss;
  parallel_ranges(n_problems, nthreads, [=](long long lo, long long hi) {
    for (long long q = lo; q < hi; ++q) {
      PcgOut o = pcg_one<T>(x + q * n, S + q * strip, Pinv + q * strip,
                            b + q * n, ss, kp, max_iters, (T)rel_tol,
                            (T)abs_tol);
      if (iters_out) iters_out[q] = o.iters;
      if (status_out) status_out[q] = o.status;
      if (rho_out) {
        rho_out[2 * q] = o.rho_init;
        rho_out[2 * q + 1] = o.rho_final;
      }
    }
  });
}

template <typename T>
void bdsv_batched(T* x, const T* S, const T* b, int ss, int kp,
                  long long n_problems, int* status_out, int nthreads) {
  const size_t strip = (size_t)kp * ss * 3 * ss, n = (size_t)kp * ss;
  parallel_ranges(n_problems, nthreads, [=](long long lo, long long hi) {
    for (long long q = lo; q < hi; ++q) {
      const int st = bdsv_one<T>(x + q * n, S + q * strip, b + q * n, ss, kp);
      if (status_out) status_out[q] = st;
    }
  });
}

}  // namespace

extern "C" {

// y (padded, [n_problems][(kp+2)*ss]) = A_bd * v; only interiors written.
void oracle_bdmv_f64(double* y, const double* S, const double* v, int ss,
                     int kp, long long n_problems, int nthreads) {
  bdmv_batched<double>(y, S, v, ss, kp, n_problems, nthreads);
}
void oracle_bdmv_f32(float* y, const float* S, const float* v, int ss, int kp,
                     long long n_problems, int nthreads) {
  bdmv_batched<float>(y, S, v, ss, kp, n_problems, nthreads);
}

// x: [n_problems][kp*ss] initial guess in, solution out.  iters/status are
// int32 [n_problems]; rho_out is [n_problems][2] = (signed rho at init,
// last rho computed).  Any of the three outputs may be NULL.
void oracle_pcg_f64(double* x, const double* S, const double* Pinv,
                    const double* b, int ss, int kp, long long n_problems,
                    int max_iters, double rel_tol, double abs_tol,
                    int* iters_out, int* status_out, double* rho_out,
                    int nthreads) {
  pcg_batched<double>(x, S, Pinv, b, ss, kp, n_problems, max_iters, rel_tol,
                      abs_tol, iters_out, status_out, rho_out, nthreads);
}
void oracle_pcg_f32(float* x, const float* S, const float* Pinv,
                    const float* b, int ss, int kp, long long n_problems,
                    int max_iters, double rel_tol, double abs_tol,
                    int* iters_out, int* status_out, double* rho_out,
                    int nthreads) {
  pcg_batched<float>(x, S, Pinv, b, ss, kp, n_problems, max_iters, rel_tol,
                     abs_tol, iters_out, status_out, rho_out, nthreads);
}

// x: [n_problems][kp*ss] solution of S x = b (left unchanged for a problem
// whose status is 1: a pivot block not numerically SPD); status: int32
// [n_problems] or NULL.
void oracle_bdsv_f64(double* x, const double* S, const double* b, int ss,
                     int kp, long long n_problems, int* status_out,
                     int nthreads) {
  bdsv_batched<double>(x, S, b, ss, kp, n_problems, status_out, nthreads);
}
void oracle_bdsv_f32(float* x, const float* S, const float* b, int ss, int kp,
                     long long n_problems, int* status_out, int nthreads) {
  bdsv_batched<float>(x, S, b, ss, kp, n_problems, status_out, nthreads);
}

// The dense n x n matrix (n = kp*ss, row-major) that one problem's strips
// stand for.  Row br*ss+i holds L_br at block-column br-1, D_br at br and
// R_br at br+1; the two blocks that fall off the matrix (L_0, R_{kp-1}) are
// dropped, which is what multiplying them by the zero pads amounts to.
void oracle_dense_expand(double* A, const double* S, int ss, int kp) {
  const int n = kp * ss, width = 3 * ss;
  for (size_t i = 0; i < (size_t)n * n; ++i) A[i] = 0.0;
  for (int br = 0; br < kp; ++br)
    for (int i = 0; i < ss; ++i) {
      const double* srow = S + ((size_t)br * ss + i) * width;
      double* arow = A + (size_t)(br * ss + i) * n;
      for (int blk = 0; blk < 3; ++blk) {
        const int bc = br - 1 + blk;  // block-column
        if (bc < 0 || bc >= kp) continue;
        for (int j = 0; j < ss; ++j) arow[bc * ss + j] = srow[blk * ss + j];
      }
    }
}

// Dense SPD solve A x = b by Cholesky (A = L L^T, Cholesky-Banachiewicz),
// forward then back substitution.  Returns 0, or -1 if a pivot is not
// positive (A not numerically SPD).
int oracle_cholesky_solve(double* x, const double* A, const double* b, int n) {
  std::vector<double> L((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j <= i; ++j) {
      double s = A[(size_t)i * n + j];
      for (int k = 0; k < j; ++k) s = s - L[(size_t)i * n + k] * L[(size_t)j * n + k];
      if (i == j) {
        if (!(s > 0.0)) return -1;
        L[(size_t)i * n + i] = std::sqrt(s);
      } else {
        L[(size_t)i * n + j] = s / L[(size_t)j * n + j];
      }
    }
  }
  std::vector<double> y(n);
  for (int i = 0; i < n; ++i) {  // L y = b
    double s = b[i];
    for (int k = 0; k < i; ++k) s = s - L[(size_t)i * n + k] * y[k];
    y[i] = s / L[(size_t)i * n + i];
  }
  for (int i = n - 1; i >= 0; --i) {  // L^T x = y
    double s = y[i];
    for (int k = i + 1; k < n; ++k) s = s - L[(size_t)k * n + i] * x[k];
    x[i] = s / L[(size_t)i * n + i];
  }
  return 0;
}

}  // extern "C"
