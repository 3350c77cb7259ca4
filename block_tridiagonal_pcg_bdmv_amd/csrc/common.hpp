// Device building blocks shared by the bdmv and PCG kernels (gfx950, wave64).
//
// * wave_sum: a 64-lane all-reduce built from DPP lane moves (quad_perm,
//   row_half_mirror, row_mirror), one ds_swizzle (xor 16 inside 32 lanes) and
//   two readlanes.  Each step adds a value to its mirror image, and IEEE
//   addition is commutative, so every lane ends with the same bits and the
//   summation tree is fixed: results are run-to-run deterministic.
// * block_sum: wave_sum, one LDS slot per wave, one barrier, then every thread
//   adds the slots in wave order -- again the same bits in every thread, so
//   scalars such as alpha, beta and the convergence test need no broadcast.
// * copy_to_lds: coalesced HBM -> LDS staging of a contiguous range with
//   16-byte loads when the caller vouches for alignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glass {

constexpr int kWave = 64;

template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// DPP control words (GCN/CDNA encoding).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <- lane 15-i within 16
constexpr int kSwizzleXor16 = 0x401F;  // ds_swizzle bitmask: and 0x1f, xor 0x10

template <int CTRL>
__device__ __forceinline__ float lane_move(float v) {
  return __int_as_float(dpp_move<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double lane_move(double v) {
  const long long bits = __double_as_longlong(v);
  const int lo = dpp_move<CTRL>((int)(bits & 0xffffffffLL));
  const int hi = dpp_move<CTRL>((int)(bits >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ float swizzle_xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
}
__device__ __forceinline__ double swizzle_xor16(double v) {
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_ds_swizzle((int)(bits & 0xffffffffLL), kSwizzleXor16);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(bits >> 32), kSwizzleXor16);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ double read_lane(double v, int lane) {
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(bits & 0xffffffffLL), lane);
  const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum over the 64 lanes of a wave; all 64 lanes must be active.  Returns the
// same value (same bits) in every lane.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v = v + lane_move<kQuadXor1>(v);
  v = v + lane_move<kQuadXor2>(v);
  v = v + lane_move<kRowHalfMirror>(v);
  v = v + lane_move<kRowMirror>(v);
  v = v + swizzle_xor16(v);
  return read_lane(v, 0) + read_lane(v, 32);
}

// s = ((slots[0] + slots[1]) + slots[2]) + ... + slots[n-1], n >= 1, the
// plain left-to-right sum, in every lane with the same bits: lane j loads
// slot j (and j + 64, ... for more than 64 slots; lanes past the end re-load
// the last slot), so one LDS round trip brings them all, and the additions
// then take the slots from the lanes one by one in order.  All 64 lanes of
// the wave must be active.
template <typename T>
__device__ __forceinline__ T sum_slots_in_order(const T* slots, int n) {
  const int lane = threadIdx.x & 63;
  T v = slots[min(lane, n - 1)];
  T s = read_lane(v, 0);
  const int n0 = min(n, 64);
  for (int c = 1; c < n0; ++c) s = s + read_lane(v, c);
  for (int base = 64; base < n; base += 64) {
    const T w = slots[min(base + lane, n - 1)];
    const int m = min(n - base, 64);
    for (int c = 0; c < m; ++c) s = s + read_lane(w, c);
  }
  return s;
}

// Workgroup-wide sum; every thread of the block must call it.  `slots` is an
// LDS array of one entry per wave that no other live block_sum is using (the
// callers alternate two arrays; a barrier separates reads of one use from
// writes of the next).  Contains exactly one __syncthreads().
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* slots, int n_waves) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) slots[wave] = v;
  __syncthreads();
  T s = slots[0];
  for (int w = 1; w < n_waves; ++w) s = s + slots[w];
  return s;
}

// Orders LDS accesses of one wave around a hand-off between its own lanes
// (DS operations of one wave execute in order; this only stops the compiler
// from moving accesses across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef float vec16_t __attribute__((ext_vector_type(4)));  // 16-byte bit copy

// Buffer resource over `nbytes` bytes at `base` (raw addressing, gfx9
// descriptor word 3).  Raw buffer loads are range-checked per dword: dwords
// at or past `nbytes` read as zero and touch no memory.
constexpr int kBufferRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes,
                                           kBufferRsrcWord3);
}
__device__ __forceinline__ vec16_t buffer_load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(vec16_t, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

// Copy `count` contiguous elements global -> LDS using `nthreads` threads
// (thread index `tid`).  With `vec`, src and dst must be 16-byte aligned; the
// bulk moves as 16-byte vectors, issued in groups so several loads are in
// flight per thread, and the tail moves element-wise.  STREAM marks data read
// once (non-temporal loads); data re-read later is loaded normally so it can
// stay in L2 / Infinity Cache.
template <bool STREAM>
__device__ __forceinline__ vec16_t load16(const vec16_t* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool STREAM, typename T>
__device__ __forceinline__ void copy_to_lds(T* __restrict__ dst,
                                            const T* __restrict__ src,
                                            int count, int tid, int nthreads,
                                            bool vec) {
  if (vec) {
    constexpr int E = 16 / sizeof(T);
    constexpr int U = 4;
    const int nv = count / E;
    const vec16_t* __restrict__ s4 = reinterpret_cast<const vec16_t*>(src);
    vec16_t* __restrict__ d4 = reinterpret_cast<vec16_t*>(dst);
    int q = tid;
    for (; q + (U - 1) * nthreads < nv; q += U * nthreads) {
      vec16_t t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = load16<STREAM>(s4 + q + u * nthreads);
#pragma unroll
      for (int u = 0; u < U; ++u) d4[q + u * nthreads] = t[u];
    }
    for (; q < nv; q += nthreads) d4[q] = load16<STREAM>(s4 + q);
    for (int e = nv * E + tid; e < count; e += nthreads) dst[e] = src[e];
  } else {
    // Element loads (unaligned source): U loads in flight before the stores.
    constexpr int U = 8;
    int e = tid;
    for (; e + (U - 1) * nthreads < count; e += U * nthreads) {
      T t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = src[e + u * nthreads];
#pragma unroll
      for (int u = 0; u < U; ++u) dst[e + u * nthreads] = t[u];
    }
    for (; e < count; e += nthreads) dst[e] = src[e];
  }
}

// Load one W-wide matrix row straight into registers.  All loads are issued
// before any is consumed, so a lane keeps W*sizeof(T) bytes in flight.  With
// WIDE the row start must be aligned to the widest power of two (<= 16 bytes)
// dividing W*sizeof(T) -- true for every row when the matrix base is 16-byte
// aligned; otherwise element loads are used.
template <typename T, int W, bool WIDE>
__device__ __forceinline__ void load_row_regs(T (&reg)[W], const T* __restrict__ src) {
  constexpr int RB = W * (int)sizeof(T);
  if constexpr (WIDE && RB % 16 == 0) {
    constexpr int NV = RB / 16, E = 16 / (int)sizeof(T);
    const vec16_t* __restrict__ s = reinterpret_cast<const vec16_t*>(src);
    vec16_t t[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) t[j] = s[j];
#pragma unroll
    for (int j = 0; j < NV; ++j) __builtin_memcpy(&reg[j * E], &t[j], 16);
  } else if constexpr (WIDE && RB % 8 == 0) {
    typedef float vec8_t __attribute__((ext_vector_type(2)));
    constexpr int NV = RB / 8, E = 8 / (int)sizeof(T);
    const vec8_t* __restrict__ s = reinterpret_cast<const vec8_t*>(src);
    vec8_t t[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) t[j] = s[j];
#pragma unroll
    for (int j = 0; j < NV; ++j) __builtin_memcpy(&reg[j * E], &t[j], 8);
  } else {
#pragma unroll
    for (int c = 0; c < W; ++c) reg[c] = src[c];
  }
}

// Debug builds (-DGLASS_AMD_LDS_NAN_FILL=1): every kernel starts by filling
// its whole dynamic LDS (`bytes` at `base`) with all-ones words, a NaN as
// float and as double, and synchronising the workgroup, so that a read of
// LDS before it is written turns the results into NaN.  Every thread of the
// workgroup must call it.  Release builds compile it to nothing.
#ifndef GLASS_AMD_LDS_NAN_FILL
#define GLASS_AMD_LDS_NAN_FILL 0
#endif
__device__ __forceinline__ void lds_debug_fill(unsigned char* base, unsigned bytes) {
#if GLASS_AMD_LDS_NAN_FILL
  unsigned* w = reinterpret_cast<unsigned*>(base);
  for (unsigned i = threadIdx.x; i < bytes / 4u; i += blockDim.x) w[i] = 0xFFFFFFFFu;
  __syncthreads();
#else
  (void)base;
  (void)bytes;
#endif
}

// Round-to-nearest a*b as its own operation (never fused into a later add).
template <typename T>
__device__ __forceinline__ T mul_unfused(T a, T b) {
#pragma clang fp contract(off)
  return a * b;
}

// Round-to-nearest a*b + c with two roundings (no contraction), for the few
// scalar decisions that must match a reference that never fuses.
template <typename T>
__device__ __forceinline__ T mul_add_unfused(T a, T b, T c) {
#pragma clang fp contract(off)
  const T m = a * b;
  return m + c;
}

template <typename T>
__device__ __forceinline__ bool is_finite_val(T v) {
  return v - v == T(0);  // false for inf and NaN
}

}  // namespace glass
