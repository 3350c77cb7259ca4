// Streaming-read rate probe (a measurement aid, not a step of the solve):
// reads a buffer once with coalesced 16-byte non-temporal loads, the access
// pattern of the bandwidth-bound kernels here, and folds every 32-bit word
// into one XOR per workgroup so the loads cannot be dropped and the result
// can be checked.  Its rate is the device's practical read ceiling, which the
// benchmark reports the HBM-bound kernels against next to the vendor peak.
#include "common.hpp"
#include "internal.hpp"

namespace glass {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread
constexpr long long kProbeChunkVecs = (long long)kProbeThreads * kProbeUnroll;

__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const vec16_t* __restrict__ src, long long nvec, unsigned* __restrict__ sink) {
  const int tid = threadIdx.x;
  unsigned acc = 0u;
  const long long nchunks = (nvec + kProbeChunkVecs - 1) / kProbeChunkVecs;
  for (long long c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const long long base = c * kProbeChunkVecs + tid;
    vec16_t t[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const long long i = base + (long long)u * kProbeThreads;
      t[u] = i < nvec ? __builtin_nontemporal_load(src + i) : vec16_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      acc ^= __float_as_uint(t[u][0]) ^ __float_as_uint(t[u][1]) ^ __float_as_uint(t[u][2]) ^
             __float_as_uint(t[u][3]);
    }
  }
  __shared__ unsigned red[kProbeThreads];
  red[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    unsigned x = 0u;
    for (int k = 0; k < kProbeThreads; ++k) x ^= red[k];
    sink[blockIdx.x] = x;
  }
}

// LDS read-rate probe (a measurement aid): each workgroup of 256 threads fills
// a 32 KB LDS buffer with word i = i * 0x9E3779B1, then every thread reads
// 16-byte vectors k = (t + 256 u + 8 r) mod 2048 for r < rounds, u < 8, and
// folds their words into an XOR; sink[w] = the XOR over the workgroup's
// threads.  WIDTH is the bytes one LDS load instruction reads per lane: 16
// (one ds_read_b128 per vector), 8 or 4 (two ds_read_b64 or four ds_read_b32,
// kept apart by volatile accesses).  The rate of the call is the LDS's read
// rate at that width.
constexpr int kLdsProbeVecs = 2048;  // 32 KB of 16-byte vectors

template <int WIDTH>
__global__ void __launch_bounds__(kProbeThreads)
lds_read_kernel(unsigned* __restrict__ sink, int rounds) {
  __shared__ vec16_t buf[kLdsProbeVecs];
  __shared__ unsigned red[kProbeThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsProbeVecs; i += kProbeThreads) {
    const unsigned w = (unsigned)i * 4u;
    buf[i] = vec16_t{__uint_as_float(w * 0x9E3779B1u), __uint_as_float((w + 1u) * 0x9E3779B1u),
                     __uint_as_float((w + 2u) * 0x9E3779B1u),
                     __uint_as_float((w + 3u) * 0x9E3779B1u)};
  }
  __syncthreads();
  unsigned acc = 0u;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = (tid + u * kProbeThreads + r * 8) & (kLdsProbeVecs - 1);
      if constexpr (WIDTH == 16) {
        const vec16_t v = buf[k];
        acc ^= __float_as_uint(v[0]) ^ __float_as_uint(v[1]) ^ __float_as_uint(v[2]) ^
               __float_as_uint(v[3]);
      } else if constexpr (WIDTH == 8) {
        typedef __attribute__((address_space(3))) const volatile unsigned long long lds_u64;
        const lds_u64* q = (const lds_u64*)(&buf[k]);
        const unsigned long long a0 = q[0], a1 = q[1];
        acc ^= (unsigned)a0 ^ (unsigned)(a0 >> 32) ^ (unsigned)a1 ^ (unsigned)(a1 >> 32);
      } else {
        typedef __attribute__((address_space(3))) const volatile unsigned lds_u32;
        const lds_u32* q = (const lds_u32*)(&buf[k]);
        acc ^= q[0] ^ q[1] ^ q[2] ^ q[3];
      }
    }
  }
  red[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    unsigned x = 0u;
    for (int k = 0; k < kProbeThreads; ++k) x ^= red[k];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

int launch_lds_read(unsigned* sink, size_t sink_words, int rounds, int width, int* workgroups,
                    hipStream_t stream) {
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  // Eight workgroups per compute unit at most, never more than the sink holds.
  long long grid = std::min<long long>(8LL * dev.cu_count, (long long)sink_words);
  if (grid < 1) grid = 1;
  auto kern = width == 16 ? lds_read_kernel<16> : width == 8 ? lds_read_kernel<8> : lds_read_kernel<4>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, sink, rounds);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "LDS read probe launch");
  *workgroups = (int)grid;
  return GLASS_OK;
}

int launch_stream_read(const void* src, size_t nbytes, unsigned* sink, size_t sink_words,
                       hipStream_t stream) {
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  const long long nvec = (long long)(nbytes / 16);
  const long long nchunks = (nvec + kProbeChunkVecs - 1) / kProbeChunkVecs;
  // Eight workgroups per compute unit at most, never more than the sink holds.
  long long grid = std::min<long long>(nchunks, 8LL * dev.cu_count);
  grid = std::min<long long>(grid, (long long)sink_words);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                     reinterpret_cast<const vec16_t*>(src), nvec, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "stream read probe launch");
  return GLASS_OK;
}

}  // namespace glass
