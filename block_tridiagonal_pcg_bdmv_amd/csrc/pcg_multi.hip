// Batched PCG with several problems per wave (GLASS user guide, page
// "Block-tridiagonal Solves", section "Solve -- glass::pcg"; the same steps,
// stopping rule and outputs as pcg_batched.hip, in another placement).
//
// For small problems (state_size 6, up to 192 rows) one problem spans LPP =
// 16 or 32 lanes, so a wave solves 64 / LPP problems at once and no
// workgroup barrier is needed: every value a problem exchanges stays inside
// its own lanes.
// * Rows are dealt interleaved: lane l of a problem owns rows l + LPP*k,
//   k < RPL, and holds their S and Pinv rows in registers for the whole
//   solve (read from memory once).  x, r, p and the transient z, S p of its
//   rows are registers too; p and r, which other lanes' matvec windows read,
//   are the problem's two padded vectors in LDS.  Lanes of one wave execute
//   their LDS operations in order, so a write followed by a wave-level
//   ordering point is visible to the other lanes' reads.
// * Dots reproduce the workgroup placement's chunk-ordered sum bit for bit.
//   There each 64-row chunk goes through the wave64 tree: pairwise sums
//   over lane distances 1, 2 (quad), the 8-lane and 16-lane mirrors, a
//   xor-16 swizzle inside 32 lanes, then lane 0 + lane 32.  With interleaved
//   rows the LPP lanes of one k form whole 16- or 32-lane groups of that
//   tree, so the DPP steps inside the group give the same partial t_k, and
//   the chunk's value is t_{2c} + t_{2c+1} (LPP = 32) or
//   (t_{4c} + t_{4c+1}) + (t_{4c+2} + t_{4c+3}) (LPP = 16), exactly the
//   swizzle and the final lane-0 + lane-32 step.  Chunks are added in
//   order.  Matvec terms run in index order with fused multiply-adds, as
//   everywhere else, so the results equal the other placements' bit for bit.
// * Problems of one wave stop at different iterations; the wave loops while
//   any of them is active and the others keep their state (their updates
//   are masked; their lanes still join the DPP steps, which never cross
//   problem boundaries).
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace glass {
namespace {

constexpr int kMultiThreads = 256;  // 4 waves; waves share nothing

template <typename T>
struct MultiArgs {
  T* x;
  const T* S;
  const T* P;
  const T* b;
  int* iters;
  int* status;
  T* rho;
  int kp;
  int n_problems;
  int max_iters;
  T rel_tol;
  T abs_tol;
  int wide;  // 16-byte aligned matrices: widest row loads
  unsigned lds_bytes;  // dynamic LDS of the launch (debug fill)
};

// Sum over the LPP lanes of one problem (all lanes of the wave take part):
// the first steps of the wave64 tree, which never cross a 16- (LPP = 16) or
// 32-lane (LPP = 32) group.  Every lane of the group gets the same bits.
template <int LPP, typename T>
__device__ __forceinline__ T group_sum(T v) {
  v = v + lane_move<kQuadXor1>(v);
  v = v + lane_move<kQuadXor2>(v);
  v = v + lane_move<kRowHalfMirror>(v);
  v = v + lane_move<kRowMirror>(v);
  if constexpr (LPP == 32) v = v + swizzle_xor16(v);
  return v;
}

template <typename T, int SS, int LPP, int RPL>
__global__ void __launch_bounds__(kMultiThreads, 2)
pcg_multi_kernel(MultiArgs<T> a) {
  constexpr int W = 3 * SS;
  constexpr int PPW = 64 / LPP;  // problems per wave
  constexpr int G = 64 / LPP;    // groups of LPP rows per 64-row chunk
  const int kp = a.kp;
  const int n = kp * SS;
  const int pad_len = (kp + 2) * SS;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int sub = lane / LPP;  // problem within the wave
  const int l = lane % LPP;
  const long long prob = ((long long)blockIdx.x * (kMultiThreads / 64) + wave) * PPW + sub;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_debug_fill(smem_raw, a.lds_bytes);
  // A wave with no problem leaves at once (wave-uniform).
  if (((long long)blockIdx.x * (kMultiThreads / 64) + wave) * PPW >= a.n_problems) return;
  const bool has_prob = prob < a.n_problems;

  T* p_pad = reinterpret_cast<T*>(smem_raw) + (size_t)(wave * PPW + sub) * 2 * pad_len;
  T* r_pad = p_pad + pad_len;

  int row[RPL], wstart[RPL];
  bool valid[RPL];
#pragma unroll
  for (int k = 0; k < RPL; ++k) {
    row[k] = l + LPP * k;
    valid[k] = has_prob && row[k] < n;
    wstart[k] = valid[k] ? (row[k] / SS) * SS : 0;
  }

  const long long mstride = (long long)n * W;
  const T* __restrict__ gS = a.S + (has_prob ? prob : 0) * mstride;
  const T* __restrict__ gP = a.P + (has_prob ? prob : 0) * mstride;
  T xr[RPL], rr[RPL], pr[RPL], tmp[RPL];
#pragma unroll
  for (int k = 0; k < RPL; ++k) {
    xr[k] = T(0);
    tmp[k] = T(0);
    if (valid[k]) {
      xr[k] = a.x[prob * n + row[k]];
      tmp[k] = a.b[prob * n + row[k]];
    }
  }
  T mS[RPL][W], mP[RPL][W];
#pragma unroll
  for (int k = 0; k < RPL; ++k) {
#pragma unroll
    for (int c = 0; c < W; ++c) {
      mS[k][c] = T(0);
      mP[k][c] = T(0);
    }
    if (valid[k]) {
      const long long off = (long long)row[k] * W;
      if (a.wide) {
        load_row_regs<T, W, true>(mS[k], gS + off);
        load_row_regs<T, W, true>(mP[k], gP + off);
      } else {
        load_row_regs<T, W, false>(mS[k], gS + off);
        load_row_regs<T, W, false>(mP[k], gP + off);
      }
    }
  }

  // out[k] = (M v)[row k]: the serial 3*ss contraction in index order.
  auto matvec = [&](const T (&m)[RPL][W], const T* __restrict__ vpad, T (&out)[RPL]) {
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      T acc = T(0);
      if (valid[k]) {
        const T* __restrict__ w = vpad + wstart[k];
#pragma unroll
        for (int c = 0; c < W; ++c) acc = fma(m[k][c], w[c], acc);
      }
      out[k] = acc;
    }
  };
  // The chunk-ordered dot (see the header): every lane of the problem gets
  // the same bits.  Rows past n (and the groups of k >= RPL inside the last
  // chunk) contribute zeros, as absent rows do in the workgroup placement.
  auto dot = [&](const T (&u)[RPL], const T (&v)[RPL]) {
    constexpr int NCH = (RPL * LPP + 63) / 64;
    T t[NCH * G];
#pragma unroll
    for (int k = 0; k < NCH * G; ++k) t[k] = T(0);
#pragma unroll
    for (int k = 0; k < RPL; ++k) t[k] = group_sum<LPP>(mul_unfused(u[k], v[k]));
    const int nchunks = (n + 63) / 64;
    T s = T(0);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      T ch;
      if constexpr (G == 2) ch = t[2 * c] + t[2 * c + 1];
      else ch = (t[4 * c] + t[4 * c + 1]) + (t[4 * c + 2] + t[4 * c + 3]);
      if (c == 0) s = ch;
      else if (c < nchunks) s = s + ch;
    }
    return s;
  };
  auto publish = [&](T* vpad, const T (&v)[RPL], bool on) {
#pragma unroll
    for (int k = 0; k < RPL; ++k)
      if (on && valid[k]) vpad[SS + row[k]] = v[k];
  };

  // Initial state: p_pad holds x0 while S x0 is formed.
  publish(p_pad, xr, true);
  for (int e = l; e < SS; e += LPP) {
    p_pad[e] = T(0);
    p_pad[(kp + 1) * SS + e] = T(0);
    r_pad[e] = T(0);
    r_pad[(kp + 1) * SS + e] = T(0);
  }
  wave_lds_sync();
  T sv[RPL];
  matvec(mS, p_pad, sv);
#pragma unroll
  for (int k = 0; k < RPL; ++k) rr[k] = valid[k] ? tmp[k] - sv[k] : T(0);
  publish(r_pad, rr, true);
  wave_lds_sync();
  matvec(mP, r_pad, sv);  // z = Pinv r
#pragma unroll
  for (int k = 0; k < RPL; ++k) pr[k] = sv[k];
  publish(p_pad, pr, true);  // p = z (the reads of x0 are done)
  T rho = dot(rr, sv);
  const T rho0 = rho;
  const T rho_init = fabs(rho);
  const T thresh = mul_add_unfused(a.rel_tol, rho_init, a.abs_tol);
  T rho_last = rho;
  int iters = 0;
  int status = GLASS_PCG_MAX_ITERS;
  bool active = has_prob;
  if (rho_init == T(0) || rho_init < thresh) {
    status = GLASS_PCG_CONVERGED;
    active = false;
  }
  wave_lds_sync();
  for (int it = 0; it < a.max_iters; ++it) {
    if (!__any(active)) break;  // wave-uniform
    matvec(mS, p_pad, sv);  // S p
    const T pSp = dot(pr, sv);
    if (active && (!(pSp > T(0)) || !is_finite_val(pSp))) {
      status = GLASS_PCG_BREAKDOWN;
      active = false;
    }
    const T alpha = rho / pSp;
    if (active) {
#pragma unroll
      for (int k = 0; k < RPL; ++k) {
        xr[k] = fma(alpha, pr[k], xr[k]);
        rr[k] = fma(-alpha, sv[k], rr[k]);
      }
      iters = it + 1;
    }
    publish(r_pad, rr, active);
    wave_lds_sync();
    matvec(mP, r_pad, sv);  // z = Pinv r
    const T rz = dot(rr, sv);
    if (active) {
      rho_last = rz;
      if (fabs(rz) < thresh) {
        status = GLASS_PCG_CONVERGED;
        active = false;
      }
    }
    const T beta = rz / rho;
    if (active) {
#pragma unroll
      for (int k = 0; k < RPL; ++k) pr[k] = fma(beta, pr[k], sv[k]);
      rho = rz;
    }
    publish(p_pad, pr, active);
    wave_lds_sync();
  }

#pragma unroll
  for (int k = 0; k < RPL; ++k)
    if (valid[k]) a.x[prob * n + row[k]] = xr[k];
  if (has_prob && l == 0) {
    if (a.iters) a.iters[prob] = iters;
    if (a.status) a.status[prob] = status;
    if (a.rho) {
      a.rho[2 * prob] = rho0;
      a.rho[2 * prob + 1] = rho_last;
    }
  }
}

// Lanes per problem and rows per lane for a state-size-6 chain of kp
// block-rows: 16 lanes up to 96 rows, 32 up to 192 (at most 6 rows per lane,
// 216 registers of matrix rows in float32, 3 rows in float64).
template <typename T>
bool multi_shape(int ss, int kp, int* lpp, int* rpl) {
  if (ss != 6) return false;
  const int n = kp * ss;
  const int max_rpl = sizeof(T) == 4 ? 6 : 3;
  for (int L : {16, 32}) {
    const int r = (n + L - 1) / L;
    if (r <= max_rpl) {
      *lpp = L;
      *rpl = r;
      return true;
    }
  }
  return false;
}

template <typename T, int LPP, int RPL>
int launch_multi_one(const MultiArgs<T>& a_in, hipStream_t st) {
  constexpr int ppb = (kMultiThreads / 64) * (64 / LPP);
  const int blocks = (a_in.n_problems + ppb - 1) / ppb;
  const size_t lds = (size_t)ppb * 2 * (a_in.kp + 2) * 6 * sizeof(T);
  MultiArgs<T> a = a_in;
  a.lds_bytes = (unsigned)lds;
  hipLaunchKernelGGL((pcg_multi_kernel<T, 6, LPP, RPL>), dim3((unsigned)blocks),
                     dim3(kMultiThreads), lds, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "pcg (several problems per wave) launch");
  return GLASS_OK;
}

template <typename T>
int launch_multi_typed(T* x, const T* S, const T* P, const T* b, int ss, int kp, int n_problems,
                       int max_iters, double rel_tol, double abs_tol, int* iters, int* status,
                       T* rho, hipStream_t st) {
  int lpp = 0, rpl = 0;
  if (!multi_shape<T>(ss, kp, &lpp, &rpl))
    return fail(GLASS_EUNSUPPORTED, "pcg: shape has no several-problems-per-wave placement");
  MultiArgs<T> a;
  a.x = x;
  a.S = S;
  a.P = P;
  a.b = b;
  a.iters = iters;
  a.status = status;
  a.rho = rho;
  a.kp = kp;
  a.n_problems = n_problems;
  a.max_iters = max_iters;
  a.rel_tol = (T)rel_tol;
  a.abs_tol = (T)abs_tol;
  const long long per = (long long)kp * ss * 3 * ss * (long long)sizeof(T);
  a.wide = aligned(S, 16) && aligned(P, 16) && per % 16 == 0;
  const int key = lpp * 10 + rpl;
  if constexpr (sizeof(T) == 4) {
    switch (key) {
      case 161: return launch_multi_one<T, 16, 1>(a, st);
      case 162: return launch_multi_one<T, 16, 2>(a, st);
      case 163: return launch_multi_one<T, 16, 3>(a, st);
      case 164: return launch_multi_one<T, 16, 4>(a, st);
      case 165: return launch_multi_one<T, 16, 5>(a, st);
      case 166: return launch_multi_one<T, 16, 6>(a, st);
      case 324: return launch_multi_one<T, 32, 4>(a, st);
      case 325: return launch_multi_one<T, 32, 5>(a, st);
      case 326: return launch_multi_one<T, 32, 6>(a, st);
      default: break;
    }
  } else {
    switch (key) {
      case 161: return launch_multi_one<T, 16, 1>(a, st);
      case 162: return launch_multi_one<T, 16, 2>(a, st);
      case 163: return launch_multi_one<T, 16, 3>(a, st);
      case 322: return launch_multi_one<T, 32, 2>(a, st);  // not reached: 16 lanes fit first
      case 323: return launch_multi_one<T, 32, 3>(a, st);
      default: break;
    }
  }
  return fail(GLASS_EUNSUPPORTED, "pcg: internal plan error (several problems per wave)");
}

}  // namespace

bool pcg_multi_fits(glass_dtype dt, int ss, int kp) {
  int lpp = 0, rpl = 0;
  return dt == GLASS_F32 ? multi_shape<float>(ss, kp, &lpp, &rpl)
                         : multi_shape<double>(ss, kp, &lpp, &rpl);
}

int launch_pcg_multi(glass_dtype dt, void* x, const void* S, const void* Pinv, const void* b,
                     int ss, int kp, int n_problems, int max_iters, double rel_tol,
                     double abs_tol, int* iters, int* status, void* rho, hipStream_t stream) {
  if (dt == GLASS_F32)
    return launch_multi_typed<float>((float*)x, (const float*)S, (const float*)Pinv,
                                     (const float*)b, ss, kp, n_problems, max_iters, rel_tol,
                                     abs_tol, iters, status, (float*)rho, stream);
  return launch_multi_typed<double>((double*)x, (const double*)S, (const double*)Pinv,
                                    (const double*)b, ss, kp, n_problems, max_iters, rel_tol,
                                    abs_tol, iters, status, (double*)rho, stream);
}

}  // namespace glass
