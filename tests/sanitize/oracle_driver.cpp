// Runs every function of the CPU oracle on small inputs (ragged sizes, one
// and several threads, NaN and non-SPD cases, zero iterations) so that an
// AddressSanitizer / UndefinedBehaviorSanitizer build reports any
// out-of-bounds access, use of uninitialised memory or undefined arithmetic.
// It checks nothing numerically (the oracle's pins do that); a clean exit is
// the result.
#include <cmath>
#include <cstdio>
#include <random>
#include <vector>

extern "C" {
void oracle_bdmv_f64(double*, const double*, const double*, int, int, long long, int);
void oracle_bdmv_f32(float*, const float*, const float*, int, int, long long, int);
void oracle_pcg_f64(double*, const double*, const double*, const double*, int, int, long long,
                    int, double, double, int*, int*, double*, int);
void oracle_pcg_f32(float*, const float*, const float*, const float*, int, int, long long, int,
                    double, double, int*, int*, double*, int);
void oracle_bdsv_f64(double*, const double*, const double*, int, int, long long, int*, int);
void oracle_bdsv_f32(float*, const float*, const float*, int, int, long long, int*, int);
void oracle_dense_expand(double*, const double*, int, int);
int oracle_cholesky_solve(double*, const double*, const double*, int);
}

namespace {

std::mt19937_64 rng(7);

// Symmetric strips with a dominant diagonal (SPD), L_{br+1} = R_br^T.
template <typename T>
std::vector<T> spd_strips(int B, int ss, int kp) {
  std::uniform_real_distribution<double> u(-0.5, 0.5);
  const int W = 3 * ss;
  std::vector<double> S((size_t)B * kp * ss * W, 0.0);
  for (int q = 0; q < B; ++q) {
    double* P = S.data() + (size_t)q * kp * ss * W;
    for (int br = 0; br + 1 < kp; ++br)
      for (int i = 0; i < ss; ++i)
        for (int j = 0; j < ss; ++j) {
          const double v = u(rng);
          P[((size_t)br * ss + i) * W + 2 * ss + j] = v;
          P[((size_t)(br + 1) * ss + j) * W + i] = v;
        }
    for (int br = 0; br < kp; ++br)
      for (int i = 0; i < ss; ++i)
        for (int j = i + 1; j < ss; ++j) {
          const double v = u(rng);
          P[((size_t)br * ss + i) * W + ss + j] = v;
          P[((size_t)br * ss + j) * W + ss + i] = v;
        }
    for (int r = 0; r < kp * ss; ++r) {
      double s = 0.0;
      for (int c = 0; c < W; ++c) s += std::fabs(P[(size_t)r * W + c]);
      P[(size_t)r * W + ss + r % ss] = s + 0.5;
    }
  }
  return std::vector<T>(S.begin(), S.end());
}

template <typename T>
std::vector<T> normals(size_t n) {
  std::normal_distribution<double> g(0.0, 1.0);
  std::vector<T> v(n);
  for (auto& e : v) e = (T)g(rng);
  return v;
}

template <typename T, typename BDMV, typename PCG, typename BDSV>
void run(BDMV bdmv, PCG pcg, BDSV bdsv) {
  const int shapes[][3] = {{1, 1, 1}, {2, 3, 4}, {5, 7, 3}, {6, 32, 5}, {3, 1, 2}, {14, 4, 2}};
  for (const auto& sh : shapes) {
    const int ss = sh[0], kp = sh[1], B = sh[2];
    const int n = kp * ss;
    auto S = spd_strips<T>(B, ss, kp);
    auto P = spd_strips<T>(B, ss, kp);
    auto v = normals<T>((size_t)B * (kp + 2) * ss);
    for (int q = 0; q < B; ++q)
      for (int e = 0; e < ss; ++e) {
        v[(size_t)q * (kp + 2) * ss + e] = 0;
        v[(size_t)q * (kp + 2) * ss + (kp + 1) * ss + e] = 0;
      }
    std::vector<T> y(v.size(), T(0));
    for (int nt : {1, 3}) bdmv(y.data(), S.data(), v.data(), ss, kp, B, nt);
    auto b = normals<T>((size_t)B * n);
    std::vector<int> it(B), st(B);
    std::vector<double> rho(2 * (size_t)B);
    for (int nt : {1, 4}) {
      for (int mi : {0, 1, 50}) {
        std::vector<T> x((size_t)B * n, T(0));
        pcg(x.data(), S.data(), P.data(), b.data(), ss, kp, B, mi, 1e-6, 0.0, it.data(),
            st.data(), rho.data(), nt);
      }
      std::vector<T> x((size_t)B * n, T(0));
      pcg(x.data(), S.data(), P.data(), b.data(), ss, kp, B, 20, 1e-6, 0.0, nullptr, nullptr,
          nullptr, nt);
      bdsv(x.data(), S.data(), b.data(), ss, kp, B, st.data(), nt);
      bdsv(x.data(), S.data(), b.data(), ss, kp, B, nullptr, nt);
    }
    // breakdown and NaN paths
    auto Sneg = S;
    for (auto& e : Sneg) e = -e;
    auto bnan = b;
    bnan[0] = (T)NAN;
    std::vector<T> x((size_t)B * n, T(0));
    pcg(x.data(), Sneg.data(), P.data(), b.data(), ss, kp, B, 20, 1e-6, 0.0, it.data(),
        st.data(), rho.data(), 2);
    pcg(x.data(), S.data(), P.data(), bnan.data(), ss, kp, B, 20, 1e-6, 0.0, it.data(),
        st.data(), rho.data(), 2);
    bdsv(x.data(), Sneg.data(), b.data(), ss, kp, B, st.data(), 2);
    // zero problems
    bdmv(y.data(), S.data(), v.data(), ss, kp, 0, 2);
    pcg(x.data(), S.data(), P.data(), b.data(), ss, kp, 0, 20, 1e-6, 0.0, it.data(), st.data(),
        rho.data(), 2);
    bdsv(x.data(), S.data(), b.data(), ss, kp, 0, st.data(), 2);
  }
}

}  // namespace

int main() {
  run<double>(oracle_bdmv_f64, oracle_pcg_f64, oracle_bdsv_f64);
  run<float>(oracle_bdmv_f32, oracle_pcg_f32, oracle_bdsv_f32);
  for (int ss : {1, 2, 3}) {
    for (int kp : {1, 2, 5}) {
      const int n = ss * kp;
      auto S = spd_strips<double>(1, ss, kp);
      std::vector<double> A((size_t)n * n), x(n);
      oracle_dense_expand(A.data(), S.data(), ss, kp);
      auto b = normals<double>(n);
      if (oracle_cholesky_solve(x.data(), A.data(), b.data(), n) != 0) return 2;
      for (auto& e : A) e = -e;
      if (oracle_cholesky_solve(x.data(), A.data(), b.data(), n) != -1) return 3;
    }
  }
  std::puts("oracle sanitizer driver: done");
  return 0;
}
