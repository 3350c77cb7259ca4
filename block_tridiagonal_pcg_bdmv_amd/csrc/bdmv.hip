// Batched block-tridiagonal matvec y = A_bd v (GLASS user guide, page
// "Block-tridiagonal Solves", sections "The [L|D|R] block-tridiagonal
// layout", "The padded vector layout" and "Matvec -- glass::bdmv").
//
// Mapping on gfx950: one workgroup owns a tile of NT consecutive strip rows
// of one problem.  The tile's rows are one contiguous range of S, so the
// workgroup stages them HBM -> LDS with 16-byte coalesced loads, stages the
// padded window of v that the tile's block-rows read, and then each thread
// owns one strip row and multiplies its 3*ss window serially (a short serial
// contraction per thread, no cross-lane reduction).  The output row
// (br+1)*ss + i of problem q is y index q*(kp+2)*ss + ss + row, so the stores
// of a wave are contiguous.  Each row is summed by one thread in a fixed
// order, so the result is independent of NT.  The operation streams S once:
// it is HBM-bandwidth bound, and the LDS hop only exists to turn the
// 3*ss-strided per-row reads into coalesced 16-byte loads.
#include <climits>

#include "common.hpp"
#include "internal.hpp"

namespace glass {
namespace {

template <typename T, int SS>
__global__ void __launch_bounds__(1024)
bdmv_kernel(T* __restrict__ y, const T* __restrict__ S,
            const T* __restrict__ v, int ss_rt, int kp,
            int tiles_per_problem, int vec) {
  const int ss = SS > 0 ? SS : ss_rt;
  const int W = 3 * ss;
  const int n = kp * ss;
  const int NT = blockDim.x;
  const int tid = threadIdx.x;
  const long long prob = blockIdx.x / tiles_per_problem;
  const int tile = (int)(blockIdx.x - prob * tiles_per_problem);
  const int row0 = tile * NT;
  const int rows = min(NT, n - row0);
  const int br_lo = row0 / ss;
  const int br_hi = (row0 + rows - 1) / ss;
  const int vcount = (br_hi - br_lo + 3) * ss;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* s_mat = reinterpret_cast<T*>(smem_raw);  // rows * W, row-major
  T* s_win = s_mat + (size_t)NT * W;          // v[br_lo*ss, (br_hi+3)*ss)

  const T* gS = S + (prob * n + row0) * (long long)W;
  copy_to_lds<true>(s_mat, gS, rows * W, tid, NT, vec != 0);
  const T* gv = v + prob * (long long)(kp + 2) * ss + (long long)br_lo * ss;
  for (int e = tid; e < vcount; e += NT) s_win[e] = gv[e];
  __syncthreads();

  if (tid < rows) {
    const int r = row0 + tid;
    const int br = r / ss;
    const T* __restrict__ m = s_mat + tid * W;
    const T* __restrict__ w = s_win + (br - br_lo) * ss;
    T acc = T(0);
    if constexpr (SS > 0) {
#pragma unroll
      for (int c = 0; c < 3 * SS; ++c) acc = fma(m[c], w[c], acc);
    } else {
      for (int c = 0; c < W; ++c) acc = fma(m[c], w[c], acc);
    }
    y[prob * (long long)(kp + 2) * ss + ss + r] = acc;
  }
}

template <typename T, int SS>
int launch_typed(T* y, const T* S, const T* v, int ss, int kp, int n_problems,
                 hipStream_t stream) {
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  const int W = 3 * ss;
  const long long n = (long long)kp * ss;
  // Threads per workgroup: 256 rows unless a tile of rows would exceed
  // ~48 KB of LDS (large state_size / fp64); never below one wave.
  int NT = (int)((48 * 1024) / ((size_t)W * sizeof(T)));
  NT = NT / 64 * 64;
  if (NT > 256) NT = 256;
  if (NT < 64) NT = 64;
  NT = env_int("GLASS_AMD_BDMV_THREADS", NT);
  if (NT % 64 != 0 || NT > 1024)
    return fail(GLASS_EINVAL, "GLASS_AMD_BDMV_THREADS must be a multiple of 64 <= 1024");
  const size_t lds = ((size_t)NT * W + NT + 4 * (size_t)ss) * sizeof(T) + 16;
  if (lds > dev.max_lds_per_block)
    return fail(GLASS_EUNSUPPORTED, "bdmv tile does not fit in LDS");
  const long long tiles = (n + NT - 1) / NT;
  const long long blocks = tiles * n_problems;
  if (blocks > INT_MAX) return fail(GLASS_EUNSUPPORTED, "bdmv grid too large");
  const int vec = aligned(S, 16) && ((n * W * (long long)sizeof(T)) % 16 == 0);
  auto kern = bdmv_kernel<T, SS>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return fail_hip(e, "hipFuncSetAttribute(bdmv)");
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), lds, stream, y, S,
                     v, ss, kp, (int)tiles, vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "bdmv launch");
  return GLASS_OK;
}

template <typename T>
int dispatch(T* y, const T* S, const T* v, int ss, int kp, int n_problems,
             hipStream_t st) {
  switch (ss) {
    case 6: return launch_typed<T, 6>(y, S, v, ss, kp, n_problems, st);
    case 12: return launch_typed<T, 12>(y, S, v, ss, kp, n_problems, st);
    case 14: return launch_typed<T, 14>(y, S, v, ss, kp, n_problems, st);
    case 21: return launch_typed<T, 21>(y, S, v, ss, kp, n_problems, st);
    default: return launch_typed<T, 0>(y, S, v, ss, kp, n_problems, st);
  }
}

}  // namespace

int launch_bdmv(glass_dtype dt, void* y, const void* S, const void* v, int ss,
                int kp, int n_problems, hipStream_t stream) {
  if (dt == GLASS_F32)
    return dispatch<float>((float*)y, (const float*)S, (const float*)v, ss, kp,
                           n_problems, stream);
  return dispatch<double>((double*)y, (const double*)S, (const double*)v, ss,
                          kp, n_problems, stream);
}

}  // namespace glass
