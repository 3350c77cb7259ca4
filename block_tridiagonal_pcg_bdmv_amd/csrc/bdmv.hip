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
// 3*ss-strided per-row reads into coalesced 16-byte loads.  For the
// specialised state sizes the tile goes from memory straight into LDS with
// direct buffer -> LDS loads (ceil(3*ss*sizeof(T)/16) 16-byte vectors per
// thread, all in flight, none through registers), marked non-temporal, through
// a buffer resource over exactly the tile's bytes: the hardware range-checks
// raw buffer loads per dword, so a tile ending inside a vector still arrives
// whole and lanes past the end read zeros, without branching.  The tile height is chosen so that the rows of a
// problem split into tiles with as little of a ragged last tile as possible.
#include <climits>

#include "common.hpp"
#include "internal.hpp"

// Tile staging for the specialised state sizes: 1 = direct buffer -> LDS
// loads (no registers in flight, no LDS stores), 0 = buffer loads into
// registers, then LDS stores.  GLASS_AMD_BDMV_AUX: cache-policy bits of the
// S loads; 2 = non-temporal (S is read once, so its lines need not stay in
// the L2 or the Infinity Cache).
#ifndef GLASS_AMD_BDMV_DIRECT
#define GLASS_AMD_BDMV_DIRECT 1
#endif
#ifndef GLASS_AMD_BDMV_AUX
#define GLASS_AMD_BDMV_AUX 2
#endif

namespace glass {
namespace {

constexpr int kBdmvMaxThreads = 256;
constexpr bool kBdmvDirect = GLASS_AMD_BDMV_DIRECT != 0;
constexpr int kBdmvAux = GLASS_AMD_BDMV_AUX;

template <typename T, int SS>
__global__ void __launch_bounds__(kBdmvMaxThreads)
bdmv_kernel(T* __restrict__ y, const T* __restrict__ S,
            const T* __restrict__ v, int ss_rt, int kp,
            int tiles_per_problem, int vec, unsigned lds_bytes) {
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
  lds_debug_fill(smem_raw, lds_bytes);
  // s_mat: rows * W matrix entries, row-major (padded to whole vectors);
  // s_win: v[br_lo*ss, (br_hi+3)*ss).
  constexpr int U = SS > 0 ? (3 * SS * (int)sizeof(T) + 15) / 16 : 1;
  T* s_mat = reinterpret_cast<T*>(smem_raw);
  T* s_win = reinterpret_cast<T*>(smem_raw + (size_t)NT * W * sizeof(T)
                                  + (SS > 0 ? (size_t)NT * (U * 16 - W * sizeof(T)) : 0));

  const T* gS = S + (prob * n + row0) * (long long)W;
  const T* gv = v + prob * (long long)(kp + 2) * ss + (long long)br_lo * ss;
  if constexpr (SS > 0) {
    const int count = rows * W;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(gS, count * (int)sizeof(T));
    if constexpr (kBdmvDirect) {
      // Vector tid + u*NT lands at the same byte offset of s_mat: a wave's
      // 64 lanes write one contiguous 1 KB per load.
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
      unsigned char* sb = reinterpret_cast<unsigned char*>(s_mat);
#pragma unroll
      for (int u = 0; u < U; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(sb + (u * NT + wave * kWave) * 16), 16,
            (tid + u * NT) * 16, 0, 0, kBdmvAux);
      for (int e = tid; e < vcount; e += NT) s_win[e] = gv[e];
      // The tile's direct loads have landed before the barrier publishes
      // them to the other waves.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      vec16_t t[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        t[u] = __builtin_bit_cast(
            vec16_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + u * NT) * 16, 0, kBdmvAux));
      for (int e = tid; e < vcount; e += NT) s_win[e] = gv[e];
      vec16_t* s4 = reinterpret_cast<vec16_t*>(s_mat);
#pragma unroll
      for (int u = 0; u < U; ++u) s4[tid + u * NT] = t[u];
    }
  } else {
    copy_to_lds<true>(s_mat, gS, rows * W, tid, NT, vec != 0);
    for (int e = tid; e < vcount; e += NT) s_win[e] = gv[e];
  }
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
  // Threads per workgroup (one per row): a multiple of 64 up to 256 rows and
  // ~48 KB of LDS, picking the height that leaves the smallest ragged last
  // tile per problem (ties: the taller tile).
  int nt_max = (int)((48 * 1024) / ((size_t)W * sizeof(T)));
  nt_max = nt_max / 64 * 64;
  if (nt_max > 256) nt_max = 256;
  if (nt_max < 64) nt_max = 64;
  int NT = 64;
  long long best_waste = -1;
  for (int c = 64; c <= nt_max; c += 64) {
    const long long waste = (n + c - 1) / c * c - n;
    if (best_waste < 0 || waste <= best_waste) {
      best_waste = waste;
      NT = c;
    }
  }
  NT = env_int("GLASS_AMD_BDMV_THREADS", NT);
  if (NT % 64 != 0 || NT > kBdmvMaxThreads)
    return fail(GLASS_EINVAL, "GLASS_AMD_BDMV_THREADS must be a multiple of 64 <= 256");
  const size_t row_bytes =
      SS > 0 ? (size_t)((W * sizeof(T) + 15) / 16 * 16) : (size_t)W * sizeof(T);
  const size_t lds = (size_t)NT * row_bytes + ((size_t)NT + 4 * (size_t)ss) * sizeof(T) + 16;
  if (lds > dev.max_lds_per_block)
    return fail(GLASS_EUNSUPPORTED, "bdmv tile does not fit in LDS");
  const long long tiles = (n + NT - 1) / NT;
  const long long blocks = tiles * n_problems;
  if (blocks > INT_MAX) return fail(GLASS_EUNSUPPORTED, "bdmv grid too large");
  const int vec = aligned(S, 16) && ((n * W * (long long)sizeof(T)) % 16 == 0);
  auto kern = bdmv_kernel<T, SS>;
  if (int rc = allow_dynamic_lds((const void*)kern, lds)) return rc;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), lds, stream, y, S,
                     v, ss, kp, (int)tiles, vec, (unsigned)lds);
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
