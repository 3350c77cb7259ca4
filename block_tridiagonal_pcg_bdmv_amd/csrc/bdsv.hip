// Batched direct solve S x = b of block-tridiagonal SPD systems (the
// glass::bdsv that the GLASS user guide page "Block-tridiagonal Solves" names
// in its opening paragraph; layout from its sections "The [L|D|R]
// block-tridiagonal layout" and "The padded vector layout").
//
// Block elimination without pivoting across block-rows (block Thomas):
//   [M_br | y_br] = [D_br | b_br] - L_br [G_{br-1} | u_{br-1}]   (br > 0)
//   [G_br | u_br] = M_br^{-1} [R_br | y_br]                      (no R_{kp-1})
//   x_{kp-1} = u_{kp-1},  x_br = u_br - G_br x_{br+1}
// M_br is a Schur complement of the SPD matrix, hence SPD; a pivot that is not
// positive marks the problem as not SPD (status 1, x left unchanged).
//
// Two mappings on gfx950, neither with workgroup barriers.
//
// Row mapping (ss <= 16; bdsv_rows_kernel): four problems per wave, one per
// 16-lane DPP row; lane i of a row holds row i of W = [M | R | y] (2ss+1
// registers).
// * Broadcasts within a problem are DPP row_newbcast:k moves, which give every
//   lane of a 16-lane row the value of lane k of that row, so four problems
//   share each instruction and no lane waits on a scalar register.
// * Fill: row i of M and y needs row i of L_br (own registers) and every row
//   of [G_{br-1} | u_{br-1}] (row m broadcast from lane m): ss*(ss+1) FMAs.
// * Gauss-Jordan without normalising the pivot row: in step k every lane
//   reads the pivot W_k[k] and subtracts (W_i[k] / W_k[k]) times the
//   broadcast pivot row from its columns > k (the pivot lane subtracts zero).
//   Rows end as piv_i [e_i | G_i | u_i] with piv_i the step-i pivot, so each
//   lane scales its [G|u] by 1/piv_i once.  About ss*(2ss+1) - ss^2/2 FMAs
//   per block-row for four problems.
// * Back substitution: lane i of a row computes x_br[i] from its row of
//   [G_br | u_br] and x_{br+1} broadcast from the row's lanes.
// * [G_br | u_br] rows go to the caller's workspace (or, without one, to
//   LDS when four problems' factors fit).  Each lane loads its own S row with
//   range-checked buffer loads (missing rows and problems read as zero), the
//   next block-row's row while the current one is eliminated.
//
// Column mapping (ss <= 24, and chains whose factors fit in LDS only for one
// problem; bdsv_kernel): one wave per problem.
// * The working block W = [M | R | y] (ss x (2ss+1)) lives in registers, one
//   column per lane: lane j holds W[0..ss)[j].
// * M^{-1} [R | y] comes from Gauss-Jordan elimination on W: ss steps; in
//   step k each lane already holds its row-k entry, and column k is read from
//   lane k with readlane into scalar registers, so the elimination touches
//   neither LDS nor memory.  Diagonal pivots are positive for SPD blocks, so
//   no row exchanges; three times fewer dependent steps than a Cholesky
//   factorisation plus two triangular solves.
// * [G_br | u_br] of every block-row is kept for the back substitution: in
//   LDS (no workspace; at most a few problems per CU fit), or in a caller's
//   workspace in HBM (WS), with only the previous block-row's [G|u] in LDS,
//   so many more problems run per CU.  The WS back substitution deals the
//   64 lanes over groups of ss lanes, each group loading one block-row's
//   rows of [G|u] (the next batch of block-rows is loaded while the current
//   one is applied), so one memory round trip covers 64/ss block-rows.
// * The next block-row's strip (ss x 3ss, one contiguous range) is
//   buffer-loaded into registers while the current block-row is eliminated,
//   then staged into LDS, where every lane reads L_br by broadcast for the
//   L_br [G|u] product.
#include <climits>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace glass {
namespace {

template <typename T>
struct BdsvArgs {
  T* x;
  const T* S;
  const T* b;
  T* ws;  // WS: [n_problems][kp][ss][ss+1] ([G_br | u_br] rows)
  int* status;
  int ss;
  int kp;
  int n_problems;
  int strip_vecs;  // 16-byte vectors per lane for one strip (LDS stage)
  unsigned lds_bytes;  // dynamic LDS of the launch (debug fill)
};

// 16-byte vectors per lane that hold one strip.
template <typename T, int SS>
constexpr int strip_slots() {
  return (3 * SS * SS * (int)sizeof(T) + 1023) / 1024;
}

template <typename T, int SS, bool WS>
__global__ void __launch_bounds__(64)
bdsv_kernel(BdsvArgs<T> a) {
  static_assert(2 * SS + 1 <= 64, "one lane per column of [M | R | y]");
  constexpr int NVS = strip_slots<T, SS>();
  constexpr int NGU = SS + 1;  // columns of [G | u]
  constexpr int SW = 3 * SS;   // strip row width
  const int kp = a.kp;
  const int lane = threadIdx.x;
  const long long prob = blockIdx.x;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_debug_fill(smem_raw, a.lds_bytes);
  T* stage = reinterpret_cast<T*>(smem_raw);            // strip: ss x 3ss (+pad)
  T* GU = stage + (size_t)NVS * 64 * (16 / sizeof(T));  // (WS ? 1 : kp) x ss x (ss+1)
  T* bv = GU + (size_t)(WS ? 1 : kp) * SS * NGU;        // b_br (ss)
  T* xbuf = bv + SS;                                    // x_{br+1} (ss)
  T* gws = WS ? a.ws + prob * (long long)kp * SS * NGU : nullptr;

  const T* gS = a.S + prob * (long long)kp * SS * SW;
  const T* gb = a.b + prob * (long long)kp * SS;

  // This lane's column of W: 0..ss-1 -> M (and G source column), ss..2ss-1
  // -> R, 2ss -> y; lanes past 2ss hold zeros and take part harmlessly.
  const int j = lane;
  const bool is_m = j < SS, is_r = j >= SS && j < 2 * SS, is_y = j == 2 * SS;

  // Strip prefetch: block-row br of S as 16-byte vectors (buffer loads over
  // exactly its bytes; dwords past the end read as zero) and b_br.
  vec16_t pf[NVS];
  T pb = T(0);
  auto prefetch = [&](int br) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(gS + (long long)br * SS * SW, SS * SW * (int)sizeof(T));
#pragma unroll
    for (int u = 0; u < NVS; ++u) pf[u] = buffer_load16(rs, (lane + u * 64) * 16);
    if (lane < SS) pb = gb[(long long)br * SS + lane];
  };
  prefetch(0);

  T w[SS];  // column j of W
  bool fail = false;
  for (int br = 0; br < kp; ++br) {
    // Stage strip br and b_br; start loading strip br+1.
    vec16_t* s4 = reinterpret_cast<vec16_t*>(stage);
#pragma unroll
    for (int u = 0; u < NVS; ++u) s4[lane + u * 64] = pf[u];
    if (lane < SS) bv[lane] = pb;
    wave_lds_sync();
    if (br + 1 < kp) prefetch(br + 1);

    // W = [D_br | R_br | b_br] - L_br [G_{br-1} | 0 | u_{br-1}], column j.
    const int c = is_m ? j : SS;  // the column of [G | u] this lane needs
    T gcol[SS];
#pragma unroll
    for (int i = 0; i < SS; ++i) {
      if (is_m) w[i] = stage[i * SW + SS + j];
      else if (is_r) w[i] = br + 1 < kp ? stage[i * SW + SS + j] : T(0);  // R: cols 2ss..3ss
      else if (is_y) w[i] = bv[i];
      else w[i] = T(0);
      gcol[i] = br > 0 ? GU[(size_t)(WS ? 0 : br - 1) * SS * NGU + i * NGU + c] : T(0);
    }
    if (br > 0 && (is_m || is_y)) {
#pragma unroll
      for (int i = 0; i < SS; ++i)
#pragma unroll
        for (int k = 0; k < SS; ++k) w[i] = fma(-stage[i * SW + k], gcol[k], w[i]);
    }

    // Gauss-Jordan: W -> [I | M^{-1} R | M^{-1} y].  Column k comes from
    // lane k (scalar registers); each lane's row-k entry is its own.
#pragma unroll
    for (int k = 0; k < SS; ++k) {
      T ck[SS];
#pragma unroll
      for (int i = 0; i < SS; ++i) ck[i] = read_lane(w[i], k);
      const T piv = ck[k];
      fail = fail || !(piv > T(0)) || !is_finite_val(piv);
      const T rk = w[k] / piv;
#pragma unroll
      for (int i = 0; i < SS; ++i) w[i] = i == k ? rk : fma(-ck[i], rk, w[i]);
    }
    if (fail) break;  // uniform over the wave

    // Keep [G_br | u_br] (columns ss .. 2ss of W): for the next block-row's
    // product (LDS) and for the back substitution (LDS or workspace).  The
    // LDS reads of the previous [G|u] above come first in program order.
    wave_lds_sync();
    if (is_r || is_y) {
      T* GUc = GU + (size_t)(WS ? 0 : br) * SS * NGU + (j - SS);
#pragma unroll
      for (int i = 0; i < SS; ++i) GUc[i * NGU] = w[i];
      if constexpr (WS) {
        T* Gg = gws + (long long)br * SS * NGU + (j - SS);
#pragma unroll
        for (int i = 0; i < SS; ++i) Gg[i * NGU] = w[i];
      }
    }
    wave_lds_sync();
  }

  if (!fail && !WS) {
    // Back substitution: x_{kp-1} = u_{kp-1}, x_br = u_br - G_br x_{br+1}.
    for (int br = kp - 1; br >= 0; --br) {
      const T* GUc = GU + (size_t)br * SS * NGU;
      T xi = T(0);
      if (lane < SS) {
        xi = GUc[lane * NGU + SS];
        if (br + 1 < kp) {
#pragma unroll
          for (int k = 0; k < SS; ++k) xi = fma(-GUc[lane * NGU + k], xbuf[k], xi);
        }
      }
      wave_lds_sync();  // every lane has read x_{br+1}
      if (lane < SS) {
        xbuf[lane] = xi;
        a.x[prob * (long long)kp * SS + (long long)br * SS + lane] = xi;
      }
      wave_lds_sync();
    }
  }
  if constexpr (WS) {
    if (!fail) {
      // Back substitution from the workspace.  Lane group g (lanes g*ss ..
      // g*ss+ss-1, NG groups) handles block-row br0 - g of the current batch;
      // lane i of the group loads row i of that block-row's [G|u].
      constexpr int NG = 64 / SS;
      const int g = lane / SS, i = lane % SS;
      const bool active = g < NG;
      // The wave's own workspace stores above must be complete and visible
      // to its other lanes before they are read back.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      T rowA[NGU], rowB[NGU];
      auto load_rows = [&](T (&row)[NGU], int br0) {
        const int br = br0 - g;
        const bool ok = active && br >= 0;
        const T* src = gws + (long long)(ok ? br : 0) * SS * NGU + i * NGU;
#pragma unroll
        for (int k = 0; k < NGU; ++k) row[k] = ok ? src[k] : T(0);
      };
      auto apply = [&](const T (&row)[NGU], int br0) {
        // Groups take their block-rows in order; x_{br+1} is in xbuf.
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const int br = br0 - gg;
          if (br < 0) break;  // uniform
          T xi = T(0);
          if (g == gg) {
            xi = row[SS];
            if (br + 1 < kp) {
#pragma unroll
              for (int k = 0; k < SS; ++k) xi = fma(-row[k], xbuf[k], xi);
            }
          }
          wave_lds_sync();  // every lane has read x_{br+1}
          if (g == gg) {
            xbuf[i] = xi;
            a.x[prob * (long long)kp * SS + (long long)br * SS + i] = xi;
          }
          wave_lds_sync();
        }
      };
      int br0 = kp - 1;
      load_rows(rowA, br0);
      while (br0 >= 0) {
        if (br0 - NG >= 0) load_rows(rowB, br0 - NG);
        apply(rowA, br0);
        br0 -= NG;
        if (br0 < 0) break;
        if (br0 - NG >= 0) load_rows(rowA, br0 - NG);
        apply(rowB, br0);
        br0 -= NG;
      }
    }
  }
  if (lane == 0 && a.status) a.status[prob] = fail ? GLASS_BDSV_NOT_SPD : GLASS_BDSV_OK;
}

// ---------------------------------------------------------------------------
// Row mapping
// ---------------------------------------------------------------------------

// Value of lane K of this lane's 16-lane row (DPP row_newbcast:K).
template <int K>
__device__ __forceinline__ int row_bcast_i32(int v) {
  static_assert(K >= 0 && K < 16, "row_newbcast lane");
  // Every source lane of a row broadcast is valid, so no old value is needed.
  return __builtin_amdgcn_mov_dpp(v, 0x150 + K, 0xF, 0xF, true);
}
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(row_bcast_i32<K>(__float_as_int(v)));
}
template <int K>
__device__ __forceinline__ double row_bcast(double v) {
  const long long bits = __double_as_longlong(v);
  const int lo = row_bcast_i32<K>((int)(bits & 0xffffffffLL));
  const int hi = row_bcast_i32<K>((int)(bits >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// 1/p: hardware reciprocal refined by Newton steps (error below one unit in
// the last place of T for normal p).
__device__ __forceinline__ float recip(float p) {
  float r = __builtin_amdgcn_rcpf(p);
  const float e = fmaf(-p, r, 1.0f);
  return fmaf(e, r, r);
}
__device__ __forceinline__ double recip(double p) {
  double r = __builtin_amdgcn_rcp(p);
  double e = fma(-p, r, 1.0);
  r = fma(e, r, r);
  e = fma(-p, r, 1.0);
  return fma(e, r, r);
}

// Buffer access of one element (range-checked; out of range reads zero and
// writes nothing).
__device__ __forceinline__ float rsrc_load(__amdgpu_buffer_rsrc_t rs, int off, float) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}
__device__ __forceinline__ double rsrc_load(__amdgpu_buffer_rsrc_t rs, int off, double) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
}
__device__ __forceinline__ void rsrc_store(__amdgpu_buffer_rsrc_t rs, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), rs, off, 0, 0);
}
__device__ __forceinline__ void rsrc_store(__amdgpu_buffer_rsrc_t rs, int off, double v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, 0);
}

constexpr int kRowsProblemsPerWave = 4;

template <typename T, int SS, bool WS>
__global__ void __launch_bounds__(64)
bdsv_rows_kernel(BdsvArgs<T> a) {
  static_assert(SS <= 16, "one 16-lane row per problem");
  constexpr int NGU = SS + 1;  // columns of [G | u]
  constexpr int NW = 2 * SS + 1;
  constexpr int SW = 3 * SS;   // S row width
  constexpr int ES = (int)sizeof(T);
  const int kp = a.kp;
  const int lane = threadIdx.x;
  const int r = lane >> 4, i = lane & 15;
  const long long p0 = (long long)blockIdx.x * kRowsProblemsPerWave;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_debug_fill(smem_raw, a.lds_bytes);
  const int nlive = (int)((long long)a.n_problems - p0 < kRowsProblemsPerWave
                              ? (long long)a.n_problems - p0
                              : kRowsProblemsPerWave);
  const long long prob = p0 + r;
  const bool act = r < nlive && i < SS;  // this lane owns row i of a problem
  const int n = kp * SS;

  // Range-checked views of this wave's problems: lanes that own no row use
  // an offset past the end, so they read zeros and write nothing.
  const int ps_bytes = n * SW * ES;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.S + p0 * n * SW, nlive * ps_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.b + p0 * n, nlive * n * ES);
  const int oS = act ? r * ps_bytes + i * SW * ES : INT_MAX / 2;
  const int ob = act ? (r * n + i) * ES : INT_MAX / 2;
  __amdgpu_buffer_rsrc_t rW = make_rsrc(a.S, 0);
  int oW = INT_MAX / 2;
  if constexpr (WS) {
    rW = make_rsrc(a.ws + p0 * n * NGU, nlive * n * NGU * ES);
    oW = act ? (r * n + i) * NGU * ES : INT_MAX / 2;
  }
  T* GUl = reinterpret_cast<T*>(smem_raw);  // !WS: [kp][4*ss][ss+1]

  T sr[SW], sb;
  auto load_row = [&](int br) {
    const int o = oS + br * SS * SW * ES;
#pragma unroll
    for (int c = 0; c < SW; ++c) sr[c] = rsrc_load(rS, o + c * ES, T(0));
    sb = rsrc_load(rb, ob + br * SS * ES, T(0));
  };
  load_row(0);

  T W[NW];
  T gp[NGU];  // this lane's row of [G_{br-1} | u_{br-1}]
#pragma unroll
  for (int j = 0; j < NGU; ++j) gp[j] = T(0);
  bool bad = false;
  for (int br = 0; br < kp; ++br) {
    // W = [D | R | b] - L [G_{br-1} | 0 | u_{br-1}]; L, D, R from the S row.
#pragma unroll
    for (int j = 0; j < SS; ++j) {
      W[j] = sr[SS + j];
      W[SS + j] = br + 1 < kp ? sr[2 * SS + j] : T(0);
    }
    W[2 * SS] = sb;
    if (br > 0) {
      static_for<0, SS>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const T nl = -sr[m];
        T t[NGU];  // row m of [G | u], issued before it is used
#pragma unroll
        for (int j = 0; j < NGU; ++j) t[j] = row_bcast<m>(gp[j]);
#pragma unroll
        for (int j = 0; j < SS; ++j) W[j] = fma(t[j], nl, W[j]);
        W[2 * SS] = fma(t[SS], nl, W[2 * SS]);
      });
    }
    if (br + 1 < kp) load_row(br + 1);

    // Gauss-Jordan without normalising the pivot row (see the file header).
    T mypiv = T(1);
    static_for<0, SS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const T piv = row_bcast<k>(W[k]);
      // The pivot row's broadcasts do not wait for the multiplier, so they
      // cover the latency of the reciprocal.
      T t[NW];
#pragma unroll
      for (int j = k + 1; j < NW; ++j) t[j] = row_bcast<k>(W[j]);
      bad = bad || !(piv > T(0)) || !is_finite_val(piv);
      mypiv = i == k ? piv : mypiv;
      const T nf = i == k ? T(0) : -(W[k] * recip(piv));
#pragma unroll
      for (int j = k + 1; j < NW; ++j) W[j] = fma(t[j], nf, W[j]);
    });
    const T inv = recip(mypiv);
#pragma unroll
    for (int j = 0; j < SS; ++j) gp[j] = W[SS + j] * inv;
    gp[SS] = W[2 * SS] * inv;

    if constexpr (WS) {
      const int o = oW + br * SS * NGU * ES;
#pragma unroll
      for (int j = 0; j < NGU; ++j) rsrc_store(rW, o + j * ES, gp[j]);
    } else {
      if (act) {
        T* dst = GUl + ((size_t)br * kRowsProblemsPerWave * SS + r * SS + i) * NGU;
#pragma unroll
        for (int j = 0; j < NGU; ++j) dst[j] = gp[j];
      }
    }
  }

  // Back substitution: x_{kp-1} = u_{kp-1}; x_br = u_br - G_br x_{br+1}.
  if constexpr (WS) {
    // This wave's workspace stores must be complete before the lanes read
    // them back.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  } else {
    wave_lds_sync();
  }
  T* gx = a.x + prob * n;
  const bool write = act && !bad;
  T xv = gp[SS];  // x_{kp-1}[i] (G_{kp-1} is zero)
  if (write) gx[(long long)(kp - 1) * SS + i] = xv;
  T rowA[NGU], rowB[NGU];
  auto load_gu = [&](T (&row)[NGU], int br) {
    if constexpr (WS) {
      const int o = oW + br * SS * NGU * ES;
#pragma unroll
      for (int j = 0; j < NGU; ++j) row[j] = rsrc_load(rW, o + j * ES, T(0));
    } else {
      const T* src = GUl + ((size_t)br * kRowsProblemsPerWave * SS + r * SS + (i < SS ? i : 0)) * NGU;
#pragma unroll
      for (int j = 0; j < NGU; ++j) row[j] = i < SS ? src[j] : T(0);
    }
  };
  auto apply = [&](const T (&row)[NGU], int br) {
    T acc0 = row[SS], acc1 = T(0);
    T xb[SS];  // x_{br+1}, one entry per lane of the row
    static_for<0, SS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      xb[j] = row_bcast<j>(xv);
    });
#pragma unroll
    for (int j = 0; j < SS; ++j) {
      if (j % 2 == 0) acc0 = fma(-row[j], xb[j], acc0);
      else acc1 = fma(-row[j], xb[j], acc1);
    }
    xv = acc0 + acc1;
    if (write) gx[(long long)br * SS + i] = xv;
  };
  int br = kp - 2;
  if (br >= 0) load_gu(rowA, br);
  while (br >= 0) {
    if (br - 1 >= 0) load_gu(rowB, br - 1);
    apply(rowA, br);
    --br;
    if (br < 0) break;
    if (br - 1 >= 0) load_gu(rowA, br - 1);
    apply(rowB, br);
    --br;
  }
  if (i == 0 && r < nlive && a.status)
    a.status[prob] = bad ? GLASS_BDSV_NOT_SPD : GLASS_BDSV_OK;
}

template <typename T, int SS, bool WS>
int launch_rows_kernel(const BdsvArgs<T>& a_in, size_t lds, hipStream_t st) {
  BdsvArgs<T> a = a_in;
  a.lds_bytes = (unsigned)lds;
  auto kern = bdsv_rows_kernel<T, SS, WS>;
  if (int rc = allow_dynamic_lds((const void*)kern, lds)) return rc;
  const unsigned grid =
      (unsigned)(((long long)a.n_problems + kRowsProblemsPerWave - 1) / kRowsProblemsPerWave);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "bdsv launch");
  return GLASS_OK;
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <typename T, int SS, bool WS>
int launch_kernel(const BdsvArgs<T>& a_in, size_t lds, hipStream_t st) {
  BdsvArgs<T> a = a_in;
  a.lds_bytes = (unsigned)lds;
  auto kern = bdsv_kernel<T, SS, WS>;
  if (int rc = allow_dynamic_lds((const void*)kern, lds)) return rc;
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_problems), dim3(64), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "bdsv launch");
  return GLASS_OK;
}

template <typename T, int SS>
int launch_typed(T* x, const T* S, const T* b, int kp, int n_problems, int* status, T* ws,
                 hipStream_t st) {
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  BdsvArgs<T> a;
  a.x = x;
  a.S = S;
  a.b = b;
  a.ws = ws;
  a.status = status;
  a.ss = SS;
  a.kp = kp;
  a.n_problems = n_problems;
  constexpr int NVS = strip_slots<T, SS>();
  a.strip_vecs = NVS;
  // Row mapping where it applies: a workspace, or four problems' factors in
  // LDS.  Byte offsets inside one wave's four problems must fit in an int.
  const bool columns = env_int("GLASS_AMD_BDSV_COLUMNS", 0) != 0;  // A/B and tests
  if constexpr (SS <= 16) {
    const double wave_bytes =
        (double)kRowsProblemsPerWave * kp * SS * 3 * SS * sizeof(T);
    const size_t rows_lds =
        ws ? 0 : (size_t)kp * kRowsProblemsPerWave * SS * (SS + 1) * sizeof(T);
    if (!columns && wave_bytes < (double)(INT_MAX / 2) && rows_lds <= dev.max_lds_per_block)
      return ws ? launch_rows_kernel<T, SS, true>(a, rows_lds, st)
                : launch_rows_kernel<T, SS, false>(a, rows_lds, st);
  }
  const size_t blocks = ws ? 1 : (size_t)kp;  // [G|u] blocks held in LDS
  const size_t lds = ((size_t)NVS * 64 * 16) + (blocks * SS * (SS + 1) + 2 * SS) * sizeof(T);
  if (lds > dev.max_lds_per_block)
    return fail(GLASS_EUNSUPPORTED,
                "bdsv: knot_points*state_size*(state_size+1) elements exceed LDS "
                "(pass a workspace)");
  return ws ? launch_kernel<T, SS, true>(a, lds, st) : launch_kernel<T, SS, false>(a, lds, st);
}

template <typename T>
int dispatch(T* x, const T* S, const T* b, int ss, int kp, int n_problems, int* status,
             T* ws, hipStream_t st) {
  switch (ss) {
#define GLASS_BDSV_CASE(N) \
  case N: return launch_typed<T, N>(x, S, b, kp, n_problems, status, ws, st);
    GLASS_BDSV_CASE(1) GLASS_BDSV_CASE(2) GLASS_BDSV_CASE(3) GLASS_BDSV_CASE(4)
    GLASS_BDSV_CASE(5) GLASS_BDSV_CASE(6) GLASS_BDSV_CASE(7) GLASS_BDSV_CASE(8)
    GLASS_BDSV_CASE(9) GLASS_BDSV_CASE(10) GLASS_BDSV_CASE(11) GLASS_BDSV_CASE(12)
    GLASS_BDSV_CASE(13) GLASS_BDSV_CASE(14) GLASS_BDSV_CASE(15) GLASS_BDSV_CASE(16)
    GLASS_BDSV_CASE(17) GLASS_BDSV_CASE(18) GLASS_BDSV_CASE(19) GLASS_BDSV_CASE(20)
    GLASS_BDSV_CASE(21) GLASS_BDSV_CASE(22) GLASS_BDSV_CASE(23) GLASS_BDSV_CASE(24)
#undef GLASS_BDSV_CASE
    default:
      return fail(GLASS_EUNSUPPORTED, "bdsv: state_size above GLASS_BDSV_MAX_STATE_SIZE");
  }
}

}  // namespace

size_t bdsv_workspace_bytes(int ss, int kp, long long n_problems, glass_dtype dt) {
  const size_t es = dt == GLASS_F32 ? sizeof(float) : sizeof(double);
  const size_t raw = (size_t)n_problems * kp * ss * (ss + 1) * es;
  return (raw + 255) & ~(size_t)255;
}

int launch_bdsv(glass_dtype dt, void* x, const void* S, const void* b, int ss, int kp,
                int n_problems, int* status, void* ws, hipStream_t stream) {
  if (dt == GLASS_F32)
    return dispatch<float>((float*)x, (const float*)S, (const float*)b, ss, kp, n_problems,
                           status, (float*)ws, stream);
  return dispatch<double>((double*)x, (const double*)S, (const double*)b, ss, kp, n_problems,
                          status, (double*)ws, stream);
}

}  // namespace glass
