// One PCG solve spread over a cooperative grid (the grid-wide PCG that the
// GLASS user guide page "Block-tridiagonal Solves" names as future work at the
// end of section "Solve -- glass::pcg").  Same steps, stopping rule and
// outputs as the batched solve; only the placement differs.
//
// Placement on one MI355X:
// * G co-resident workgroups; workgroup g owns block-rows [A, B) (nb = B - A
//   >= 2).  Partition indices are dealt so that consecutive partitions sit on
//   the same XCD (workgroups are dispatched round-robin over the 8 XCDs), so
//   most neighbour exchanges stay inside one XCD's L2.
// * Ghost zones.  Each workgroup also computes S p and the r update for the
//   block-rows A-1 and B ("extended rows"), and keeps p for A-2 .. B+1.  The
//   ghost values are computed with exactly the same fused operations as their
//   owners, so they are bit-identical copies.  After the r^T z reduction the
//   owners publish z of their two edge block-rows on each side; neighbours
//   rebuild p = z + beta p on the ghosts themselves.  That leaves two grid
//   barriers per iteration -- one per dot product -- and no separate halo
//   exchange step.
// * Grid dot (grid_dot): per-thread partial -> wave64 DPP tree -> LDS slot
//   per wave -> wave 0 adds the wave slots in order and publishes the
//   workgroup partial (and the edge z values staged in LDS).  The workgroups
//   form (up to) 8 groups of consecutive partitions -- one group per XCD.  A
//   workgroup arrives at its group counter; the last arriver of a group (known
//   from the fetch-add result) adds the group's partials in partition order,
//   publishes the group sum and arrives at the top counter.  Every workgroup
//   waits for the top counter, loads the group sums and adds them in group
//   order, so every workgroup holds identical alpha, beta and stopping
//   decisions.  Only wave 0 of a workgroup takes part.
// * Publication without cache maintenance: every value another workgroup
//   reads (partials, group sums, edge z) is written with device-scope
//   atomic stores and read with device-scope atomic loads, which the
//   hardware serves at the device coherence point; the writing wave waits for
//   its stores to complete (s_waitcnt vmcnt(0)) before it arrives.  A
//   device-scope release/acquire fence instead writes back / invalidates the
//   XCD's L2, which costs several microseconds per barrier and grows with
//   the number of workgroups.
// * Matrices: for the specialised state sizes each thread keeps its S row
//   (extended rows) and Pinv row (own rows) in VGPRs, loaded once with every
//   load of the row in flight; the iteration then touches only registers,
//   LDS and the small exchange buffers.
// * Grid barrier: monotonically increasing arrival counters (group and
//   top), polled by one lane with relaxed loads and s_sleep between polls.
//   The poll is bounded: a timeout sets a flag, every later wait returns as
//   soon as it sees the flag, the kernel runs to its end, and the status
//   output reports the timeout instead of the device hanging.
#include <climits>

#include "common.hpp"
#include "internal.hpp"

namespace glass {
namespace {

constexpr int kGridMaxWorkgroups = 2048;
constexpr unsigned kSpinLimit = 1u << 21;

template <typename T>
struct GridArgs {
  T* x;
  const T* S;
  const T* P;
  const T* b;
  int* iters;
  int* status;
  T* rho;
  int ss;
  int kp;
  int max_iters;
  T rel_tol;
  T abs_tol;
  unsigned int* counter;  // top-level arrivals (zeroed before the launch)
  unsigned int* flags;    // [0]: a barrier wait timed out
  unsigned int* gcount;   // group arrivals, one per kCounterStride words
  T* gsum1;               // [kGroups] group sums of the p^T S p partials
  T* gsum2;               // [kGroups] group sums of the r^T z partials
  T* slot1;               // [G] per-workgroup p^T S p partials
  T* slot2;               // [G] per-workgroup r^T z partials
  T* edges;               // [G][4*ss]: z of block-rows A, A+1, B-2, B-1
  int G;
  int nb_max;
  int wide;               // matrix bases 16-byte aligned: vector row loads
};

// Barrier groups (one per XCD) and the spacing of their counters (one
// 128-byte cache line each).
constexpr int kGroups = 8;
constexpr int kCounterStride = 32;

struct WorkspaceLayout {
  size_t counter, gcount, gsum1, gsum2, slot1, slot2, edges, total;
};

inline size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

WorkspaceLayout layout(int ss, int kp, size_t elem) {
  const size_t gmax = (size_t)std::min(kp / 2, kGridMaxWorkgroups);
  WorkspaceLayout w;
  w.counter = 0;  // counter at +0, flags at +4
  w.gcount = 256;
  w.gsum1 = w.gcount + kGroups * kCounterStride * sizeof(unsigned int);
  w.gsum2 = w.gsum1 + 256;
  w.slot1 = w.gsum2 + 256;
  w.slot2 = w.slot1 + round256(gmax * elem);
  w.edges = w.slot2 + round256(gmax * elem);
  w.total = w.edges + round256(gmax * 4 * (size_t)ss * elem);
  return w;
}

__global__ void grid_reset_kernel(unsigned int* counter, unsigned int* gcount) {
  if (threadIdx.x < 2) counter[threadIdx.x] = 0u;  // counter, flags[0]
  if (threadIdx.x < kGroups) gcount[threadIdx.x * kCounterStride] = 0u;
}

template <typename T>
__device__ __forceinline__ T load_shared_global(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ void store_shared_global(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's earlier global stores have completed.
__device__ __forceinline__ void wait_stores_complete() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Poll `counter` until it reaches `target` (one lane).  Bounded: see the
// timeout rule at the top of the file.
__device__ __forceinline__ void wait_counter(const unsigned int* counter,
                                             unsigned int target,
                                             unsigned int* flags) {
  unsigned int spins = 0;
  while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 255u) == 0u &&
        __hip_atomic_load(flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
      break;  // another workgroup already gave up: do not wait again
    if (spins > kSpinLimit) {
      __hip_atomic_store(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// Partials one lane loads per batch in the group sum.
constexpr int kSumBatch = 8;

// Where the barrier groups split the G partitions: group k holds partitions
// [group_begin(k), group_begin(k+1)).
__device__ __forceinline__ int group_begin(int k, int G, int ngroups) {
  return (int)((long long)k * G / ngroups);
}

struct GridSync {
  unsigned int* counter;
  unsigned int* gcount;
  unsigned int* flags;
  int g, G, ngroups, grp, gbeg, gsize;
};

// Grid-wide sum of the per-thread values v; every thread of every workgroup
// must call it and gets the same bits.  If `edge_lds` is non-null, wave 0
// also publishes the workgroup's n_edge edge z values staged there.  `bar`
// is the barrier number (1-based).  Contains two __syncthreads().
template <typename T>
__device__ __forceinline__ T grid_dot(T v, T* __restrict__ slots, T* __restrict__ gsum,
                                      const T* edge_lds, T* __restrict__ edges_g,
                                      int n_edge, const GridSync& gs, unsigned int bar,
                                      T* wsl, T* bcast, int NW, int wave, int lane) {
  v = wave_sum(v);
  if (lane == 0) wsl[wave] = v;
  __syncthreads();
  if (wave == 0) {
    T part = wsl[0];
    for (int w = 1; w < NW; ++w) part = part + wsl[w];
    if (edge_lds)
      for (int j = lane; j < n_edge; j += kWave) store_shared_global(edges_g + j, edge_lds[j]);
    if (lane == 0) store_shared_global(slots + gs.g, part);
    wait_stores_complete();
    unsigned int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(gs.gcount + gs.grp * kCounterStride, 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == bar * (unsigned)gs.gsize - 1u) {
      // Last arriver of the group: every member's partial is published.
      // Add them in partition order (lane-strided, then the wave tree).
      T s = T(0);
      for (int base = 0; base < gs.gsize; base += kSumBatch * kWave) {
        T val[kSumBatch];
#pragma unroll
        for (int k = 0; k < kSumBatch; ++k) {
          const int j = base + lane + k * kWave;
          val[k] = j < gs.gsize ? load_shared_global(slots + gs.gbeg + j) : T(0);
        }
#pragma unroll
        for (int k = 0; k < kSumBatch; ++k)
          if (base + lane + k * kWave < gs.gsize) s = s + val[k];
      }
      s = wave_sum(s);
      if (lane == 0) store_shared_global(gsum + gs.grp, s);
      wait_stores_complete();
      if (lane == 0)
        __hip_atomic_fetch_add(gs.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) wait_counter(gs.counter, bar * (unsigned)gs.ngroups, gs.flags);
    // Group sums in group order (every lane loads all of them).
    T gv[kGroups];
#pragma unroll
    for (int k = 0; k < kGroups; ++k)
      gv[k] = k < gs.ngroups ? load_shared_global(gsum + k) : T(0);
    T t = gv[0];
#pragma unroll
    for (int k = 1; k < kGroups; ++k)
      if (k < gs.ngroups) t = t + gv[k];
    if (lane == 0) *bcast = t;
  }
  __syncthreads();
  return *bcast;
}

template <typename T, int SS, bool RES>
__global__ void __launch_bounds__(RES ? 512 : 1024)
pcg_grid_kernel(GridArgs<T> a) {
  constexpr int WC = SS > 0 ? 3 * SS : 1;
  const int ss = SS > 0 ? SS : a.ss;
  const int W = 3 * ss;
  const int kp = a.kp;
  const int G = a.G;
  const int NT = blockDim.x;
  const int NW = NT >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int bid = blockIdx.x;
  const int g = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int A = (int)((long long)g * kp / G);
  const int B = (int)((long long)(g + 1) * kp / G);
  const int nb = B - A;
  const int next = (nb + 2) * ss;  // extended rows: block-rows A-1 .. B
  const int loc_len = (a.nb_max + 4) * ss;
  const int n_edge = 4 * ss;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* p_loc = reinterpret_cast<T*>(smem_raw);  // block-rows A-2 .. B+1
  T* r_loc = p_loc + loc_len;                 // same indexing
  T* edge_lds = r_loc + loc_len;              // [4*ss] z of A, A+1, B-2, B-1
  T* wsl = edge_lds + n_edge;                 // [NW]
  T* bcast = wsl + NW;                        // [1]

  // This thread's extended row.
  const int e = tid;
  const int br = A - 1 + (e < next ? e / ss : 0);
  const int i = e < next ? e % ss : 0;
  const bool valid = e < next && br >= 0 && br < kp;
  const bool own = valid && br >= A && br < B;
  const long long grow = (long long)br * ss + i;
  const int wstart = (e < next ? e / ss : 0) * ss;  // window start in p_loc/r_loc

  // z of a block-row outside [A, B), as published by its owner (0 outside).
  auto ghost_z = [&](int gbr, int gi) -> T {
    if (gbr < 0 || gbr >= kp) return T(0);
    if (gbr < A) return load_shared_global(a.edges + (size_t)(g - 1) * n_edge + 2 * ss +
                                           (gbr - (A - 2)) * ss + gi);
    return load_shared_global(a.edges + (size_t)(g + 1) * n_edge + (gbr - B) * ss + gi);
  };
  // Owners of the two edge block-rows on each side stage their z in LDS;
  // wave 0 publishes the array inside the next grid_dot.
  auto stage_edges = [&](T zval) {
    if (!own) return;
    if (br < A + 2) edge_lds[(br - A) * ss + i] = zval;
    if (br >= B - 2) edge_lds[2 * ss + (br - (B - 2)) * ss + i] = zval;
  };
  GridSync gs;
  gs.counter = a.counter;
  gs.gcount = a.gcount;
  gs.flags = a.flags;
  gs.g = g;
  gs.G = G;
  gs.ngroups = G < kGroups ? G : kGroups;
  gs.grp = 0;
  while (gs.grp + 1 < gs.ngroups && group_begin(gs.grp + 1, G, gs.ngroups) <= g) ++gs.grp;
  gs.gbeg = group_begin(gs.grp, G, gs.ngroups);
  gs.gsize = group_begin(gs.grp + 1, G, gs.ngroups) - gs.gbeg;
  unsigned int barriers = 0;
  auto dot = [&](T v, T* slots, T* gsum, bool with_edges) {
    ++barriers;
    return grid_dot(v, slots, gsum, with_edges ? edge_lds : (const T*)nullptr,
                    a.edges + (size_t)g * n_edge, n_edge, gs, barriers, wsl, bcast,
                    NW, wave, lane);
  };

  // Matrix rows in registers (specialised sizes): S for every valid extended
  // row, Pinv for owned rows.
  T mS[WC], mP[WC];
  if constexpr (RES) {
#pragma unroll
    for (int c = 0; c < WC; ++c) {
      mS[c] = T(0);
      mP[c] = T(0);
    }
    if (valid) {
      if (a.wide) load_row_regs<T, WC, true>(mS, a.S + grow * WC);
      else load_row_regs<T, WC, false>(mS, a.S + grow * WC);
    }
    if (own) {
      if (a.wide) load_row_regs<T, WC, true>(mP, a.P + grow * WC);
      else load_row_regs<T, WC, false>(mP, a.P + grow * WC);
    }
  }
  auto row_dot = [&](const T* __restrict__ gM, const T* __restrict__ mreg,
                     const T* __restrict__ vloc) -> T {
    T acc = T(0);
    const T* __restrict__ w = vloc + wstart;
    if constexpr (RES) {
#pragma unroll
      for (int c = 0; c < WC; ++c) acc = fma(mreg[c], w[c], acc);
    } else {
      const T* __restrict__ m = gM + grow * W;
      for (int c = 0; c < W; ++c) acc = fma(m[c], w[c], acc);
    }
    return acc;
  };

  // Initial state: p_loc holds x0 on block-rows A-2 .. B+1 (0 off the chain).
  for (int j = tid; j < (nb + 4) * ss; j += NT) {
    const int gbr = A - 2 + j / ss;
    p_loc[j] = (gbr >= 0 && gbr < kp) ? a.x[(long long)gbr * ss + j % ss] : T(0);
    r_loc[j] = T(0);
  }
  T xr = own ? a.x[grow] : T(0);
  const T bb = valid ? a.b[grow] : T(0);
  __syncthreads();

  T sv = valid ? row_dot(a.S, mS, p_loc) : T(0);
  T rr = valid ? bb - sv : T(0);
  if (e < next) r_loc[e + ss] = rr;
  __syncthreads();
  T z = own ? row_dot(a.P, mP, r_loc) : T(0);
  stage_edges(z);
  T rho = dot(own ? rr * z : T(0), a.slot2, a.gsum2, true);
  const T rho0 = rho;
  const T rho_init = fabs(rho);
  const T thresh = mul_add_unfused(a.rel_tol, rho_init, a.abs_tol);
  T rho_last = rho;
  int iters = 0;
  int status = GLASS_PCG_MAX_ITERS;
  T pr = T(0);
  if (rho_init == T(0) || rho_init < thresh) {
    status = GLASS_PCG_CONVERGED;
  } else {
    // p = z on the extended rows and the two outer ghost block-rows.
    pr = valid ? (own ? z : ghost_z(br, i)) : T(0);
    if (e < next) p_loc[e + ss] = pr;
    if (tid < ss) p_loc[tid] = ghost_z(A - 2, tid);
    else if (tid < 2 * ss) p_loc[(nb + 3) * ss + tid - ss] = ghost_z(B + 1, tid - ss);
    __syncthreads();

    for (int it = 0; it < a.max_iters; ++it) {
      sv = valid ? row_dot(a.S, mS, p_loc) : T(0);  // S p on extended rows
      const T pSp = dot(own ? pr * sv : T(0), a.slot1, a.gsum1, false);
      if (!(pSp > T(0)) || !is_finite_val(pSp)) {
        status = GLASS_PCG_BREAKDOWN;
        break;
      }
      const T alpha = rho / pSp;
      if (own) xr = fma(alpha, pr, xr);
      if (valid) rr = fma(-alpha, sv, rr);
      if (e < next) r_loc[e + ss] = rr;
      iters = it + 1;
      __syncthreads();
      z = own ? row_dot(a.P, mP, r_loc) : T(0);
      stage_edges(z);
      const T rz = dot(own ? rr * z : T(0), a.slot2, a.gsum2, true);
      rho_last = rz;
      if (fabs(rz) < thresh) {
        status = GLASS_PCG_CONVERGED;
        break;
      }
      const T beta = rz / rho;
      if (valid) {
        const T zext = own ? z : ghost_z(br, i);
        pr = fma(beta, pr, zext);
      }
      if (e < next) p_loc[e + ss] = pr;
      if (tid < ss) p_loc[tid] = fma(beta, p_loc[tid], ghost_z(A - 2, tid));
      else if (tid < 2 * ss)
        p_loc[(nb + 3) * ss + tid - ss] =
            fma(beta, p_loc[(nb + 3) * ss + tid - ss], ghost_z(B + 1, tid - ss));
      rho = rz;
      __syncthreads();
    }
  }

  if (iters > 0 && own) a.x[grow] = xr;
  if (g == 0 && tid == 0) {
    const bool timed_out =
        __hip_atomic_load(a.flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    if (a.iters) a.iters[0] = iters;
    if (a.status) a.status[0] = timed_out ? GLASS_PCG_GRID_TIMEOUT : status;
    if (a.rho) {
      a.rho[0] = rho0;
      a.rho[1] = rho_last;
    }
  }
}

template <typename T, int SS, bool RES>
int launch_grid_typed(GridArgs<T> a, int NT, size_t lds, const DeviceInfo& dev,
                      hipStream_t st) {
  auto kern = pcg_grid_kernel<T, SS, RES>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return fail_hip(e, "hipFuncSetAttribute(grid)");
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NT, lds);
  if (e != hipSuccess) return fail_hip(e, "occupancy query (grid)");
  if ((long long)per_cu * dev.cu_count < a.G)
    return fail(GLASS_ECOOP, "grid pcg: workgroups cannot all be co-resident");
  hipLaunchKernelGGL(grid_reset_kernel, dim3(1), dim3(64), 0, st, a.counter, a.gcount);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "grid reset launch");
  void* args[] = {&a};
  e = hipLaunchCooperativeKernel((const void*)kern, dim3(a.G), dim3(NT), args,
                                 (unsigned)lds, st);
  if (e == hipErrorCooperativeLaunchTooLarge)
    return fail(GLASS_ECOOP, "grid pcg: cooperative launch too large");
  if (e != hipSuccess) return fail_hip(e, "grid pcg cooperative launch");
  return GLASS_OK;
}

// Register-resident S and Pinv rows (3*ss each) within the 256-VGPR budget of
// a 512-thread workgroup, leaving room for the solver state.
template <typename T>
constexpr bool kGridResidentFits(int ss) {
  return 6 * ss * (int)sizeof(T) / 4 <= 160;
}

template <typename T, int SS>
int launch_grid_res(GridArgs<T> a, int NT, size_t lds, const DeviceInfo& dev,
                    hipStream_t st) {
  if constexpr (kGridResidentFits<T>(SS)) return launch_grid_typed<T, SS, true>(a, NT, lds, dev, st);
  return fail(GLASS_EUNSUPPORTED, "grid pcg: internal plan error");
}

template <typename T>
int launch_grid(T* x, const T* S, const T* P, const T* b, int ss, int kp,
                int max_iters, double rel_tol, double abs_tol, int* iters,
                int* status, T* rho, void* workspace, size_t ws_bytes,
                hipStream_t st) {
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  if (!dev.cooperative)
    return fail(GLASS_ECOOP, "device does not support cooperative launches");
  const WorkspaceLayout wl = layout(ss, kp, sizeof(T));
  if (ws_bytes < wl.total)
    return fail(GLASS_EINVAL, "grid pcg: workspace too small");
  const bool specialised = ss == 6 || ss == 12 || ss == 14 || ss == 21;
  const bool res = specialised && kGridResidentFits<T>(ss);
  const int max_threads = res ? 512 : 1024;
  const int gmax = std::min(kp / 2, kGridMaxWorkgroups);
  // One workgroup per CU to start; more only if a partition would need more
  // rows than one workgroup holds.
  int G = std::min(gmax, dev.cu_count);
  G = env_int("GLASS_AMD_GRID_WGS", G);
  if (G < 1 || G > gmax)
    return fail(GLASS_EINVAL, "GLASS_AMD_GRID_WGS out of range");
  int nb_max = 0, NT = 0;
  for (;;) {
    nb_max = (kp + G - 1) / G;
    NT = ((nb_max + 2) * ss + 63) / 64 * 64;
    if (NT < 2 * ss) NT = (2 * ss + 63) / 64 * 64;
    if (NT <= max_threads) break;
    if (G >= gmax)
      return fail(GLASS_EUNSUPPORTED, "grid pcg: chain too long for the grid");
    G = std::min(gmax, G * 2);
  }
  // The group counters count up to (2*max_iters + 1) * (group size) without
  // wrapping (the group size is at most G).
  if ((2.0 * max_iters + 1.0) * G >= (double)UINT_MAX)
    return fail(GLASS_EUNSUPPORTED, "grid pcg: max_iters too large for the barrier counter");
  const int NW = NT / 64;
  const size_t loc_len = (size_t)(nb_max + 4) * ss;
  const size_t lds = (2 * loc_len + 4 * (size_t)ss + NW + 1) * sizeof(T);
  if (lds > dev.max_lds_per_block)
    return fail(GLASS_EUNSUPPORTED, "grid pcg: partition does not fit in LDS");

  GridArgs<T> a;
  a.x = x;
  a.S = S;
  a.P = P;
  a.b = b;
  a.iters = iters;
  a.status = status;
  a.rho = rho;
  a.ss = ss;
  a.kp = kp;
  a.max_iters = max_iters;
  a.rel_tol = (T)rel_tol;
  a.abs_tol = (T)abs_tol;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.counter = reinterpret_cast<unsigned int*>(ws + wl.counter);
  a.flags = a.counter + 1;
  a.gcount = reinterpret_cast<unsigned int*>(ws + wl.gcount);
  a.gsum1 = reinterpret_cast<T*>(ws + wl.gsum1);
  a.gsum2 = reinterpret_cast<T*>(ws + wl.gsum2);
  a.slot1 = reinterpret_cast<T*>(ws + wl.slot1);
  a.slot2 = reinterpret_cast<T*>(ws + wl.slot2);
  a.edges = reinterpret_cast<T*>(ws + wl.edges);
  a.G = G;
  a.nb_max = nb_max;
  a.wide = aligned(S, 16) && aligned(P, 16);
  if (res) {
    switch (ss) {
      case 6: return launch_grid_res<T, 6>(a, NT, lds, dev, st);
      case 12: return launch_grid_res<T, 12>(a, NT, lds, dev, st);
      case 14: return launch_grid_res<T, 14>(a, NT, lds, dev, st);
      default: return launch_grid_res<T, 21>(a, NT, lds, dev, st);
    }
  }
  return launch_grid_typed<T, 0, false>(a, NT, lds, dev, st);
}

}  // namespace

size_t grid_workspace_bytes(int ss, int kp, glass_dtype dt) {
  return layout(ss, kp, dt == GLASS_F32 ? sizeof(float) : sizeof(double)).total;
}

int launch_pcg_grid(glass_dtype dt, void* x, const void* S, const void* Pinv,
                    const void* b, int ss, int kp, int max_iters,
                    double rel_tol, double abs_tol, int* iters, int* status,
                    void* rho, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  if (dt == GLASS_F32)
    return launch_grid<float>((float*)x, (const float*)S, (const float*)Pinv,
                              (const float*)b, ss, kp, max_iters, rel_tol,
                              abs_tol, iters, status, (float*)rho, workspace,
                              workspace_bytes, stream);
  return launch_grid<double>((double*)x, (const double*)S, (const double*)Pinv,
                             (const double*)b, ss, kp, max_iters, rel_tol,
                             abs_tol, iters, status, (double*)rho, workspace,
                             workspace_bytes, stream);
}

}  // namespace glass
