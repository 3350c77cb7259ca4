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
// Mapping on gfx950: one wave per problem (no workgroup barriers at all).
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

template <typename T, int SS, bool WS>
int launch_kernel(const BdsvArgs<T>& a, size_t lds, hipStream_t st) {
  auto kern = bdsv_kernel<T, SS, WS>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return fail_hip(e, "hipFuncSetAttribute(bdsv)");
  }
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
  constexpr int NVS = strip_slots<T, SS>();
  const size_t blocks = ws ? 1 : (size_t)kp;  // [G|u] blocks held in LDS
  const size_t lds = ((size_t)NVS * 64 * 16) + (blocks * SS * (SS + 1) + 2 * SS) * sizeof(T);
  if (lds > dev.max_lds_per_block)
    return fail(GLASS_EUNSUPPORTED,
                "bdsv: knot_points*state_size*(state_size+1) elements exceed LDS "
                "(pass a workspace)");
  BdsvArgs<T> a;
  a.x = x;
  a.S = S;
  a.b = b;
  a.ws = ws;
  a.status = status;
  a.ss = SS;
  a.kp = kp;
  a.n_problems = n_problems;
  a.strip_vecs = NVS;
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
