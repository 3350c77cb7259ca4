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
//   per wave -> wave 0 adds the wave slots in order, giving the workgroup
//   partial.  Exchange through tagged words: every value another workgroup
//   reads is published as 64-bit words [tag | 32 bits of the value] (one
//   word per float, two per double), where the tag is the barrier's number
//   within the solve.  A 64-bit store is single-copy atomic, so a reader that
//   sees the expected tag also sees the value stored with it; no counter,
//   fence or store-completion wait is needed.  Wave 0 stores the partial
//   (and the workgroup's edge z values), then loads all G partials -- and
//   the neighbours' edge z values -- until every tag is current, and adds the
//   partials in a fixed lane-strided order followed by the wave tree.  Every
//   workgroup runs the same summation, so all hold identical alpha, beta and
//   stopping decisions.  One store and about one load round trip per dot,
//   against the five dependent round trips of a counter-based two-level
//   barrier (measured 2.2 us against 4.4 us per barrier at 256 workgroups).
// * Partial copies.  Each partial is stored into kPartCopies copies of the
//   partial array, and a workgroup polls copy blockIdx % kPartCopies: the
//   workgroups of one XCD share a copy, so each line is polled by G/8
//   workgroups instead of G.  The same values are added in the same order
//   whichever copy is read.  Measured at 256 workgroups: fp64 chain 81-82 ->
//   73 us, fp32 47-48 -> 43.5 us (16 or more copies were slower than 8).
//   Each partial also has a slot of its own of kSlotBytes, so two
//   workgroups at most store into one 128-byte line (fp64 chain a further
//   72.7 -> 68.5 us).
// * Staggered polls.  Wave 0 keeps two poll rounds of the partials in
//   flight, half a round trip apart, and checks them alternately (where the
//   second set of words fits in registers): fp32 chain 42.7 -> 38.7 us,
//   fp64 73.8 -> 72.0 us.
// * Reuse rules.  Partials and edge values alternate between two buffers by
//   barrier parity: a workgroup writes the buffers of barrier n+2 only after
//   it has seen every partial of barrier n+1, and each of those was stored
//   after its writer had finished reading barrier n (its edge loads
//   included).  One buffer would do for edges published every other barrier
//   (the standard steps), not for the single-reduction form, which publishes
//   them at every barrier.
//   Tags are relative to a per-solve base: barrier b is tagged base + b.  By
//   default a reset kernel zeroes the words the solve reads and the base is 1.
//   When the caller keeps the workspace for grid solves only
//   (GLASS_GRID_KEEP_WORKSPACE, and always for the static no-alloc scratch),
//   the host hands each solve a base above every tag an earlier solve could
//   have written there (a solve has at most 2 max_iters + 2 barriers), so
//   stale words never match and no reset is launched; the whole area is
//   zeroed once, on first use of the address and before the 32-bit tags
//   would wrap.
// * Matrices: for the specialised state sizes each thread keeps its S row
//   (extended rows) and Pinv row (own rows) in VGPRs, loaded once with every
//   load of the row in flight; the iteration then touches only registers,
//   LDS and the small exchange buffers.
// * Bounded polls: a poll that exceeds its spin limit sets a flag, every
//   other poll stops as soon as it sees the flag, the kernel runs to its end,
//   and the status output reports the timeout instead of the device hanging.
#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"
#include "internal.hpp"

namespace glass {
namespace {

constexpr int kGridMaxWorkgroups = 2048;
// Poll rounds before a wait gives up (GLASS_AMD_GRID_SPIN_LIMIT overrides it,
// which lets tests drive the timeout path from the host).
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
  unsigned int* flags;       // [0]: a poll timed out (zeroed before the launch)
  unsigned long long* part;  // [kPartCopies][2][G][kSlotWords] tagged partials, by barrier parity
  unsigned long long* edges; // [2][G][4*ss][kTagWords<T>] tagged edge values (block-rows
                             // A, A+1, B-2, B-1), by barrier parity
  int G;
  int nb_max;
  int wide;               // matrix bases 16-byte aligned: vector row loads
  unsigned spin_limit;    // poll rounds before a wait gives up
  unsigned tag_base;      // barrier b of this solve is tagged tag_base + b; a
                          // timeout stores tag_base into flags[0]
  unsigned lds_bytes;     // dynamic LDS of the launch (debug fill)
};

typedef unsigned long long u64;

// 64-bit exchange words per value: one for float, two for double.
template <typename T>
constexpr int kTagWords = (int)sizeof(T) / 4;

// Values one grid dot can reduce at once (the single-reduction variant
// reduces two).
constexpr int kDotValues = 2;

// Copies of the partial array (see "Partial copies" at the top of the file).
constexpr int kPartCopies = 8;
static_assert(kPartCopies <= 64, "one wave stores every copy");
// Bytes of one workgroup's slot in a partial array (its NV values, padded).
constexpr int kSlotBytes = 64;
static_assert(kDotValues * 2 * 8 <= kSlotBytes, "a slot holds every value of a dot");
constexpr int kSlotWords = kSlotBytes / 8;

struct WorkspaceLayout {
  size_t flags, part, edges, total;
};

inline size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// Exchange area for a grid of G workgroups.
WorkspaceLayout layout_for(size_t G, int ss, size_t elem) {
  const size_t words = elem / 4;
  WorkspaceLayout w;
  w.flags = 0;
  w.part = 256;
  w.edges = w.part + round256((size_t)kPartCopies * 2 * G * kSlotBytes);
  w.total = w.edges + round256(2 * G * 4 * (size_t)ss * words * sizeof(u64));
  return w;
}

// A caller's workspace is sized for the largest grid a chain of kp
// block-rows can take, so it serves every device.
WorkspaceLayout layout(int ss, int kp, size_t elem) {
  return layout_for((size_t)std::min(kp / 2, kGridMaxWorkgroups), ss, elem);
}

// The exchange area of glass_pcg_grid_noalloc: one array per device that
// holds the library's code, kept until the process ends.  Host code never
// passes the array's name to a kernel (in host code it is only a stand-in
// for the symbol); it passes the device address that hipGetSymbolAddress
// returns for the current device, taken once per device.
constexpr size_t kNoAllocScratchBytes = GLASS_PCG_GRID_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;  // by device ordinal; null until first used

int scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((int)g_scratch_ptr.size() <= device) g_scratch_ptr.resize(device + 1, nullptr);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(grid scratch)");
    if (!p) return fail(GLASS_EHIP, "hipGetSymbolAddress(grid scratch) returned NULL");
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return GLASS_OK;
}

// Zeroes the timeout flag and tag words: n1 words at w1 and n2 words at w2
// (the partial buffers and edges the solve reads, or the whole area).
__global__ void grid_reset_kernel(unsigned int* flags, u64* w1, long long n1, u64* w2,
                                  long long n2) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  if (i == 0) flags[0] = 0u;
  for (long long j = i; j < n1; j += stride) w1[j] = 0ull;
  for (long long j = i; j < n2; j += stride) w2[j] = 0ull;
}

// Tag epochs of kept exchange areas, by (device, address): the next free tag
// base, valid only after the whole area was zeroed (every word there is then
// zero or a tag below it).
struct Epoch {
  unsigned next = 0;
};
std::mutex g_epoch_mutex;
std::map<std::pair<int, uintptr_t>, Epoch> g_epochs;
constexpr unsigned long long kTagLimit = 0xFFFFFF00ull;

enum ResetKind { kResetNone = 0, kResetRegion = 1, kResetAll = 2 };
struct EpochPlan {
  unsigned base = 1;
  ResetKind reset = kResetRegion;
};

// Barriers one solve can use: the standard steps 1 + 2 max_iters, the
// single-reduction form max_iters + 2.
inline unsigned long long barrier_bound(int max_iters) {
  return 2ull * (unsigned long long)max_iters + 2ull;
}

EpochPlan epoch_begin(int device, const void* area, bool keep, int max_iters) {
  EpochPlan p;
  const auto key = std::make_pair(device, reinterpret_cast<uintptr_t>(area));
  std::lock_guard<std::mutex> lock(g_epoch_mutex);
  if (!keep) {
    g_epochs.erase(key);  // the caller may change the area before a later kept solve
    return p;             // zero what this solve reads, tags from 1
  }
  auto it = g_epochs.find(key);
  if (it != g_epochs.end() &&
      (unsigned long long)it->second.next + barrier_bound(max_iters) + 1ull < kTagLimit) {
    p.base = it->second.next;
    p.reset = kResetNone;
  } else {
    p.reset = kResetAll;
  }
  return p;
}

void epoch_commit(int device, const void* area, bool keep, int max_iters, const EpochPlan& p) {
  if (!keep) return;
  const auto key = std::make_pair(device, reinterpret_cast<uintptr_t>(area));
  const unsigned long long next = (unsigned long long)p.base + barrier_bound(max_iters) + 1ull;
  std::lock_guard<std::mutex> lock(g_epoch_mutex);
  if (next >= kTagLimit) {
    g_epochs.erase(key);
  } else {
    g_epochs[key].next = (unsigned)next;
  }
}

__device__ __forceinline__ u64 load_word(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_word(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish v as kTagWords<T> words [tag | 32 value bits], low half first.
__device__ __forceinline__ void put_tagged(u64* dst, float v, unsigned tag) {
  store_word(dst, ((u64)tag << 32) | __float_as_uint(v));
}
__device__ __forceinline__ void put_tagged(u64* dst, double v, unsigned tag) {
  const u64 bits = (u64)__double_as_longlong(v);
  store_word(dst, ((u64)tag << 32) | (bits & 0xffffffffull));
  store_word(dst + 1, ((u64)tag << 32) | (bits >> 32));
}

// Read a value published by put_tagged; true if every word carries `tag`.
__device__ __forceinline__ bool get_tagged(const u64* src, unsigned tag, float& out) {
  const u64 w = load_word(src);
  out = __uint_as_float((unsigned)w);
  return (unsigned)(w >> 32) == tag;
}
__device__ __forceinline__ bool get_tagged(const u64* src, unsigned tag, double& out) {
  const u64 w0 = load_word(src);
  const u64 w1 = load_word(src + 1);
  out = __longlong_as_double((long long)((w1 << 32) | (w0 & 0xffffffffull)));
  return ((unsigned)(w0 >> 32) == tag) & ((unsigned)(w1 >> 32) == tag);
}

// One more round of a bounded poll by a whole wave (see the timeout rule at
// the top of the file); false when the poll must stop.  The flag holds the
// tag base of the solve that timed out, so a flag left by an earlier solve
// never stops this one.
__device__ __forceinline__ bool keep_polling(unsigned& spins, unsigned int* flags, int lane,
                                             unsigned limit, unsigned tag_base) {
  __builtin_amdgcn_s_sleep(1);
  ++spins;
  if ((spins & 63u) == 0u &&
      __hip_atomic_load(flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag_base)
    return false;  // another workgroup already gave up: do not wait again
  if (spins > limit) {
    if (lane == 0) __hip_atomic_store(flags, tag_base, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  return true;
}

// Partials one lane loads per poll round.
constexpr int kSumBatch = 4;
// Sleep units (64 clocks) between the two poll rounds of a grid dot.
constexpr int kPollStagger = 20;

// The value of kTagWords<T> exchange words read raw (see put_tagged).
template <typename T>
__device__ __forceinline__ T tagged_value(const u64 (&w)[kTagWords<T>]) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float((unsigned)w[0]);
  } else {
    return __longlong_as_double((long long)((w[1] << 32) | (w[0] & 0xffffffffull)));
  }
}

// Where a workgroup's exchange buffers are (edge pointers for parity 0; the
// parity-1 buffers follow at edge_parity words).
struct GridXchg {
  u64* part;         // [kPartCopies][2][G][kSlotWords]
  u64* my_edges;     // this workgroup's [4*ss][kTagWords]
  const u64* left;   // left neighbour's edges, or null (first partition)
  const u64* right;  // right neighbour's edges, or null (last partition)
  size_t edge_parity;
  unsigned int* flags;
  unsigned spin_limit;
  unsigned tag_base;
  int G, g;
  int copy;  // the partial copy this workgroup polls
};

// Grid-wide sums of NV per-thread values v[0..NV); every thread of every
// workgroup must call it and gets the same bits in out[0..NV).  `bar` is the
// barrier number (1-based, the same sequence in every workgroup).  With
// edge_lds, wave 0 also publishes this workgroup's n_edge = 4*ss edge values
// staged there and fills ghost_lds with the neighbours' ones: [0, 2ss) of
// block-rows A-2, A-1 and [2ss, 4ss) of B, B+1 (zero off the chain).  GP
// bounds the ghost values per lane (GP*64 >= n_edge).  Contains two
// __syncthreads().
template <typename T, int GP, int NV, bool STAGGER>
__device__ __forceinline__ void grid_dot_n(const T (&v)[NV], T (&out)[NV], const T* edge_lds,
                                           T* ghost_lds, int n_edge, const GridXchg& xc,
                                           unsigned bar, T* wsl, T* bcast, int NW, int wave,
                                           int lane) {
  static_assert(NV >= 1 && NV <= kDotValues, "values per grid dot");
  constexpr int WD = kTagWords<T>;
  const unsigned tag = xc.tag_base + bar;
  T vs[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) vs[q] = wave_sum(v[q]);
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < NV; ++q) wsl[q * NW + wave] = vs[q];
  }
  __syncthreads();
  if (wave == 0) {
    // The workgroup's partials, its waves' sums added in wave order (all
    // slots in one LDS round trip).
    T part[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) part[q] = sum_slots_in_order(wsl + q * NW, NW);
    // Partial array of copy c for this barrier's parity.
    auto slots_of = [&](int c) {
      return xc.part + ((size_t)c * 2 + (bar & 1u)) * xc.G * kSlotWords;
    };
    const size_t epar = (bar & 1u) ? xc.edge_parity : 0;
    const u64* left = xc.left ? xc.left + epar : nullptr;
    const u64* right = xc.right ? xc.right + epar : nullptr;
    if (edge_lds)
      for (int j = lane; j < n_edge; j += kWave)
        put_tagged(xc.my_edges + epar + j * WD, edge_lds[j], tag);
    if (lane < kPartCopies) {  // lane c stores into copy c
      u64* mine = slots_of(lane) + xc.g * kSlotWords;
#pragma unroll
      for (int q = 0; q < NV; ++q) put_tagged(mine + q * WD, part[q], tag);
    }
    const u64* slots = slots_of(xc.copy);

    // Neighbour edges: loaded now, checked after the partials, so both
    // share one round trip when the neighbours are on time.
    const int half = n_edge >> 1;
    T gv[GP];
    bool gok = true;
    if (edge_lds) {
#pragma unroll
      for (int k = 0; k < GP; ++k) {
        const int q = lane + k * kWave;
        gv[k] = T(0);
        if (q < n_edge) {
          const u64* src = q < half ? left : right;
          if (src) gok &= get_tagged(src + (q < half ? q + half : q - half) * WD, tag, gv[k]);
        }
      }
    }

    // All G partials, polled in batches until every tag is current, added in
    // a fixed order: lane-strided within the batch sequence, then the tree.
    T sum[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) sum[q] = T(0);
    if constexpr (STAGGER) {
      // Two poll rounds in flight, started kPollStagger sleep units (64
      // clocks each) apart and re-issued alternately: a partial that lands
      // just after one round's load is seen by the other round about half a
      // round trip later instead of a whole one.  The same words are added
      // in the same order.  The caller picks it where the second set of
      // words does not make its kernel spill.
      for (int base = 0; base < xc.G; base += kSumBatch * kWave) {
        u64 wa[kSumBatch][NV][WD], wb[kSumBatch][NV][WD];
        auto issue = [&](u64 (&w)[kSumBatch][NV][WD]) {
#pragma unroll
          for (int k = 0; k < kSumBatch; ++k) {
            const int j = base + lane + k * kWave;
#pragma unroll
            for (int q = 0; q < NV; ++q)
#pragma unroll
              for (int d = 0; d < WD; ++d)  // entries past G read as current
                w[k][q][d] = j < xc.G ? load_word(slots + j * kSlotWords + q * WD + d)
                                      : ((u64)tag << 32);
          }
        };
        auto ready = [&](const u64 (&w)[kSumBatch][NV][WD]) {
          bool ok = true;
#pragma unroll
          for (int k = 0; k < kSumBatch; ++k)
#pragma unroll
            for (int q = 0; q < NV; ++q)
#pragma unroll
              for (int d = 0; d < WD; ++d) ok &= (unsigned)(w[k][q][d] >> 32) == tag;
          return __all(ok);
        };
        auto add = [&](const u64 (&w)[kSumBatch][NV][WD]) {
#pragma unroll
          for (int k = 0; k < kSumBatch; ++k)
            if (base + lane + k * kWave < xc.G) {
#pragma unroll
              for (int q = 0; q < NV; ++q) sum[q] = sum[q] + tagged_value<T>(w[k][q]);
            }
        };
        unsigned spins = 0;
        issue(wa);
        __builtin_amdgcn_s_sleep(kPollStagger);
        issue(wb);
        for (;;) {
          if (ready(wa) || !keep_polling(spins, xc.flags, lane, xc.spin_limit, xc.tag_base)) {
            add(wa);
            break;
          }
          issue(wa);
          if (ready(wb) || !keep_polling(spins, xc.flags, lane, xc.spin_limit, xc.tag_base)) {
            add(wb);
            break;
          }
          issue(wb);
        }
      }
    } else
    for (int base = 0; base < xc.G; base += kSumBatch * kWave) {
      T val[kSumBatch][NV];
      unsigned spins = 0;
      for (;;) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < kSumBatch; ++k) {
          const int j = base + lane + k * kWave;
#pragma unroll
          for (int q = 0; q < NV; ++q) {
            val[k][q] = T(0);
            if (j < xc.G) ok &= get_tagged(slots + j * kSlotWords + q * WD, tag, val[k][q]);
          }
        }
        if (__all(ok)) break;
        if (!keep_polling(spins, xc.flags, lane, xc.spin_limit, xc.tag_base)) break;
      }
#pragma unroll
      for (int k = 0; k < kSumBatch; ++k)
        if (base + lane + k * kWave < xc.G) {
#pragma unroll
          for (int q = 0; q < NV; ++q) sum[q] = sum[q] + val[k][q];
        }
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) sum[q] = wave_sum(sum[q]);

    if (edge_lds) {
      unsigned spins = 0;
      while (!__all(gok)) {
        if (!keep_polling(spins, xc.flags, lane, xc.spin_limit, xc.tag_base)) break;
        gok = true;
#pragma unroll
        for (int k = 0; k < GP; ++k) {
          const int q = lane + k * kWave;
          if (q < n_edge) {
            const u64* src = q < half ? left : right;
            if (src) gok &= get_tagged(src + (q < half ? q + half : q - half) * WD, tag, gv[k]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < GP; ++k)
        if (lane + k * kWave < n_edge) ghost_lds[lane + k * kWave] = gv[k];
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < NV; ++q) bcast[q] = sum[q];
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NV; ++q) out[q] = bcast[q];
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
  lds_debug_fill(smem_raw, a.lds_bytes);
  T* p_loc = reinterpret_cast<T*>(smem_raw);  // block-rows A-2 .. B+1
  T* r_loc = p_loc + loc_len;                 // same indexing
  T* edge_lds = r_loc + loc_len;              // [4*ss] z of A, A+1, B-2, B-1
  T* ghost_lds = edge_lds + n_edge;           // [4*ss] z of A-2, A-1, B, B+1
  T* wsl = ghost_lds + n_edge;                // [kDotValues][NW]
  T* bcast = wsl + kDotValues * NW;           // [kDotValues]

  // This thread's extended row.
  const int e = tid;
  const int br = A - 1 + (e < next ? e / ss : 0);
  const int i = e < next ? e % ss : 0;
  const bool valid = e < next && br >= 0 && br < kp;
  const bool own = valid && br >= A && br < B;
  const long long grow = (long long)br * ss + i;
  const int wstart = (e < next ? e / ss : 0) * ss;  // window start in p_loc/r_loc
  // A whole number of 16-byte vectors per block: say so, so the window reads
  // can be 16-byte LDS loads.
  if constexpr (SS > 0 && (SS * sizeof(T)) % 16 == 0)
    __builtin_assume((wstart & (int)(16 / sizeof(T) - 1)) == 0);

  // z of a block-row outside [A, B) (A-2, A-1, B or B+1), as received from
  // its owner in the last r^T z dot (0 off the chain).
  auto ghost_z = [&](int gbr, int gi) -> T {
    return gbr < A ? ghost_lds[(gbr - (A - 2)) * ss + gi] : ghost_lds[2 * ss + (gbr - B) * ss + gi];
  };
  // Owners of the two edge block-rows on each side stage their z in LDS;
  // wave 0 publishes the array inside the next grid_dot.
  auto stage_edges = [&](T zval) {
    if (!own) return;
    if (br < A + 2) edge_lds[(br - A) * ss + i] = zval;
    if (br >= B - 2) edge_lds[2 * ss + (br - (B - 2)) * ss + i] = zval;
  };
  constexpr int WD = kTagWords<T>;
  constexpr int GP = SS > 0 ? (4 * SS + kWave - 1) / kWave : (4 * 64 + kWave - 1) / kWave;
  GridXchg xc;
  xc.part = a.part;
  xc.my_edges = a.edges + (size_t)g * n_edge * WD;
  xc.left = g > 0 ? a.edges + (size_t)(g - 1) * n_edge * WD : nullptr;
  xc.right = g + 1 < G ? a.edges + (size_t)(g + 1) * n_edge * WD : nullptr;
  xc.edge_parity = (size_t)G * n_edge * WD;
  xc.spin_limit = a.spin_limit;
  xc.tag_base = a.tag_base;
  xc.flags = a.flags;
  xc.G = G;
  xc.g = g;
  xc.copy = bid % kPartCopies;
  unsigned int barriers = 0;
  auto dot = [&](T v, bool with_edges) {
    ++barriers;
    T in[1] = {v}, out[1];
    grid_dot_n<T, GP, 1, true>(in, out, with_edges ? edge_lds : (const T*)nullptr, ghost_lds,
                               n_edge, xc, barriers, wsl, bcast, NW, wave, lane);
    return out[0];
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
      // Where a block is a whole number of 16-byte vectors (see wstart),
      // every window starts 16-byte aligned (each vector is nb_max + 4
      // blocks from an aligned base) and is read with 16-byte LDS loads.
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
  T rho = dot(own ? rr * z : T(0), true);
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
      const T pSp = dot(own ? pr * sv : T(0), false);
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
      const T rz = dot(own ? rr * z : T(0), true);
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
        __hip_atomic_load(a.flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.tag_base;
    if (a.iters) a.iters[0] = iters;
    if (a.status) a.status[0] = timed_out ? GLASS_PCG_GRID_TIMEOUT : status;
    if (a.rho) {
      a.rho[0] = rho0;
      a.rho[1] = rho_last;
    }
  }
}

// Single-reduction PCG over the same placement (the communication-reducing
// form of Chronopoulos and Gear, preconditioned as written out by Ghysels and
// Vanroose): in exact arithmetic the same iterates, stopping rule and
// iteration count as the standard steps, with r^T u and w^T u reduced in one
// grid dot, so one grid barrier per iteration instead of two (the rounding
// differs).  u = Pinv r, w = S u, and further recurrence vectors replace the
// second dot:
//   r0 = b - S x0; u0 = Pinv r0; w0 = S u0
//   for i = 0, 1, ...:  gamma = r^T u; delta = w^T u       (one reduction)
//     stop when |gamma| < thresh (i updates done) or i = max_iters
//     m = Pinv w; n = S m
//     beta = gamma / gamma_prev (0 at i = 0)
//     d = delta - beta gamma / alpha_prev (delta at i = 0)  [= p^T S p]
//     d not positive: breakdown; alpha = gamma / d
//     z = n + beta z; q = m + beta q; s = w + beta s; p = u + beta p
//     x += alpha p; r -= alpha s; u -= alpha q; w -= alpha z
// Each workgroup keeps Pinv rows for its extended rows A-1 .. B as well, so
// m is computed there and n = S m needs no exchange; the reduction carries the
// owners' w of their two edge block-rows on each side.  One more exchange at
// the start carries u0's edges for w0.
template <typename T, int SS, bool RES>
__global__ void __launch_bounds__(RES ? 512 : 1024)
pcg_grid_cg1_kernel(GridArgs<T> a) {
  constexpr int WC = SS > 0 ? 3 * SS : 1;
  const int ss = SS > 0 ? SS : a.ss;
  const int W = 3 * ss;
  const int kp = a.kp;
  const int G = a.G;
  const int NT = blockDim.x;
  const int NW = NT >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int g = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int A = (int)((long long)g * kp / G);
  const int B = (int)((long long)(g + 1) * kp / G);
  const int nb = B - A;
  const int next = (nb + 2) * ss;  // extended rows: block-rows A-1 .. B
  const int loc_len = (a.nb_max + 4) * ss;
  const int n_edge = 4 * ss;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_debug_fill(smem_raw, a.lds_bytes);
  T* w_loc = reinterpret_cast<T*>(smem_raw);  // block-rows A-2 .. B+1
  T* m_loc = w_loc + loc_len;                 // same indexing
  T* edge_lds = m_loc + loc_len;              // [4*ss] values of A, A+1, B-2, B-1
  T* ghost_lds = edge_lds + n_edge;           // [4*ss] values of A-2, A-1, B, B+1
  T* wsl = ghost_lds + n_edge;                // [kDotValues][NW]
  T* bcast = wsl + kDotValues * NW;           // [kDotValues]

  const int e = tid;
  const int br = A - 1 + (e < next ? e / ss : 0);
  const int i = e < next ? e % ss : 0;
  const bool valid = e < next && br >= 0 && br < kp;
  const bool own = valid && br >= A && br < B;
  const long long grow = (long long)br * ss + i;
  const int wstart = (e < next ? e / ss : 0) * ss;
  if constexpr (SS > 0 && (SS * sizeof(T)) % 16 == 0)
    __builtin_assume((wstart & (int)(16 / sizeof(T) - 1)) == 0);

  auto ghost = [&](int gbr, int gi) -> T {
    return gbr < A ? ghost_lds[(gbr - (A - 2)) * ss + gi] : ghost_lds[2 * ss + (gbr - B) * ss + gi];
  };
  auto stage_edges = [&](T val) {
    if (!own) return;
    if (br < A + 2) edge_lds[(br - A) * ss + i] = val;
    if (br >= B - 2) edge_lds[2 * ss + (br - (B - 2)) * ss + i] = val;
  };
  // Fill a window vector on block-rows A-2 .. B+1 from this workgroup's own
  // values and the neighbours' edges.
  auto fill_window = [&](T* loc, T own_val) {
    if (e < next) loc[e + ss] = valid ? (own ? own_val : ghost(br, i)) : T(0);
    if (tid < ss) loc[tid] = ghost(A - 2, tid);
    else if (tid < 2 * ss) loc[(nb + 3) * ss + tid - ss] = ghost(B + 1, tid - ss);
  };
  constexpr int GP = SS > 0 ? (4 * SS + kWave - 1) / kWave : (4 * 64 + kWave - 1) / kWave;
  constexpr int WD = kTagWords<T>;
  GridXchg xc;
  xc.part = a.part;
  xc.my_edges = a.edges + (size_t)g * n_edge * WD;
  xc.left = g > 0 ? a.edges + (size_t)(g - 1) * n_edge * WD : nullptr;
  xc.right = g + 1 < G ? a.edges + (size_t)(g + 1) * n_edge * WD : nullptr;
  xc.edge_parity = (size_t)G * n_edge * WD;
  xc.spin_limit = a.spin_limit;
  xc.tag_base = a.tag_base;
  xc.flags = a.flags;
  xc.G = G;
  xc.g = g;
  xc.copy = bid % kPartCopies;
  unsigned int barriers = 0;
  auto dot2 = [&](T v0, T v1, T (&out)[2]) {
    ++barriers;
    T in[2] = {v0, v1};
    // Staggered polls: fp32 up to state size 14 (fp64, and larger states,
    // would spill the second set of words).
    constexpr bool kStagger = sizeof(T) == 4 && (SS > 0 && SS <= 14);
    grid_dot_n<T, GP, 2, kStagger>(in, out, edge_lds, ghost_lds, n_edge, xc, barriers, wsl,
                                   bcast, NW, wave, lane);
  };

  // S and Pinv rows of every valid extended row.
  T mS[WC], mP[WC];
  if constexpr (RES) {
#pragma unroll
    for (int c = 0; c < WC; ++c) {
      mS[c] = T(0);
      mP[c] = T(0);
    }
    if (valid) {
      if (a.wide) {
        load_row_regs<T, WC, true>(mS, a.S + grow * WC);
        load_row_regs<T, WC, true>(mP, a.P + grow * WC);
      } else {
        load_row_regs<T, WC, false>(mS, a.S + grow * WC);
        load_row_regs<T, WC, false>(mP, a.P + grow * WC);
      }
    }
  }
  auto row_dot = [&](const T* __restrict__ gM, const T* __restrict__ mreg,
                     const T* __restrict__ vloc) -> T {
    T acc = T(0);
    const T* __restrict__ w = vloc + wstart;
    if constexpr (RES) {
      // Where a block is a whole number of 16-byte vectors (see wstart),
      // every window starts 16-byte aligned (each vector is nb_max + 4
      // blocks from an aligned base) and is read with 16-byte LDS loads.
#pragma unroll
      for (int c = 0; c < WC; ++c) acc = fma(mreg[c], w[c], acc);
    } else {
      const T* __restrict__ m = gM + grow * W;
      for (int c = 0; c < W; ++c) acc = fma(m[c], w[c], acc);
    }
    return acc;
  };

  // r0 on the extended rows from x0 on A-2 .. B+1 (w_loc), u0 on own rows.
  for (int j = tid; j < (nb + 4) * ss; j += NT) {
    const int gbr = A - 2 + j / ss;
    w_loc[j] = (gbr >= 0 && gbr < kp) ? a.x[(long long)gbr * ss + j % ss] : T(0);
    m_loc[j] = T(0);
  }
  T xr = own ? a.x[grow] : T(0);
  const T bb = valid ? a.b[grow] : T(0);
  __syncthreads();
  T rr = valid ? bb - row_dot(a.S, mS, w_loc) : T(0);
  if (e < next) m_loc[e + ss] = rr;
  __syncthreads();
  T uu = own ? row_dot(a.P, mP, m_loc) : T(0);
  // Exchange u0's edges (the sums are not used), then w0 = S u0.
  stage_edges(uu);
  T red[2];
  dot2(own ? rr * uu : T(0), T(0), red);
  fill_window(w_loc, uu);
  __syncthreads();
  T ww = own ? row_dot(a.S, mS, w_loc) : T(0);

  T zz = T(0), qq = T(0), sv = T(0), pp = T(0);
  T rho0 = T(0), rho_last = T(0), thresh = T(0);
  T gamma_prev = T(1), alpha_prev = T(1);
  int iters = 0;
  int status = GLASS_PCG_MAX_ITERS;
  for (int it = 0;; ++it) {
    stage_edges(ww);
    dot2(own ? rr * uu : T(0), own ? ww * uu : T(0), red);
    const T gamma = red[0], delta = red[1];
    rho_last = gamma;
    if (it == 0) {
      rho0 = gamma;
      const T rho_init = fabs(gamma);
      thresh = mul_add_unfused(a.rel_tol, rho_init, a.abs_tol);
      if (rho_init == T(0) || rho_init < thresh) {
        status = GLASS_PCG_CONVERGED;
        break;
      }
    } else if (fabs(gamma) < thresh) {
      status = GLASS_PCG_CONVERGED;
      break;
    }
    if (it >= a.max_iters) break;  // GLASS_PCG_MAX_ITERS
    // m = Pinv w on the extended rows, n = S m on own rows.
    fill_window(w_loc, ww);
    __syncthreads();
    const T mm = valid ? row_dot(a.P, mP, w_loc) : T(0);
    if (e < next) m_loc[e + ss] = mm;
    __syncthreads();
    const T nn = own ? row_dot(a.S, mS, m_loc) : T(0);
    const T beta = it == 0 ? T(0) : gamma / gamma_prev;
    const T d = it == 0 ? delta : delta - beta * gamma / alpha_prev;
    if (!(d > T(0)) || !is_finite_val(d)) {
      status = GLASS_PCG_BREAKDOWN;
      break;
    }
    const T alpha = gamma / d;
    if (own) {
      zz = fma(beta, zz, nn);
      qq = fma(beta, qq, mm);
      sv = fma(beta, sv, ww);
      pp = fma(beta, pp, uu);
      xr = fma(alpha, pp, xr);
      rr = fma(-alpha, sv, rr);
      uu = fma(-alpha, qq, uu);
      ww = fma(-alpha, zz, ww);
    }
    gamma_prev = gamma;
    alpha_prev = alpha;
    iters = it + 1;
  }

  if (iters > 0 && own) a.x[grow] = xr;
  if (g == 0 && tid == 0) {
    const bool timed_out =
        __hip_atomic_load(a.flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.tag_base;
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
                      bool exclusive, bool single, void* area, size_t area_bytes, bool keep,
                      hipStream_t st) {
  auto kern = single ? pcg_grid_cg1_kernel<T, SS, RES> : pcg_grid_kernel<T, SS, RES>;
  if (int rc = allow_dynamic_lds((const void*)kern, lds)) return rc;
  int per_cu = 0;
  if (int rc = kernel_occupancy((const void*)kern, NT, lds, &per_cu)) return rc;
  hipError_t e = hipSuccess;
  if ((long long)per_cu * dev.cu_count < a.G)
    return fail(GLASS_ECOOP, "grid pcg: workgroups cannot all be co-resident");
  a.lds_bytes = (unsigned)lds;
  // Tag base and reset (see the exchange rules at the top of the file).
  const EpochPlan ep = epoch_begin(dev.device, area, keep, a.max_iters);
  a.tag_base = ep.base;
  if (ep.reset != kResetNone) {
    long long n1, n2;
    u64* w1;
    if (ep.reset == kResetAll) {  // the whole area
      w1 = reinterpret_cast<u64*>(area);
      n1 = (long long)(area_bytes / sizeof(u64));
      n2 = 0;
    } else {  // the words this grid reads: both partial buffers and the edges
      w1 = a.part;
      n1 = (long long)kPartCopies * 2 * a.G * kSlotWords;
      n2 = 2LL * a.G * 4 * a.ss * kTagWords<T>;
    }
    const long long most = std::max(n1, n2);
    const int reset_blocks = (int)std::min<long long>(1024, (most + 255) / 256);
    hipLaunchKernelGGL(grid_reset_kernel, dim3(reset_blocks), dim3(256), 0, st, a.flags, w1, n1,
                       a.edges, n2);
    e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "grid reset launch");
  }
  void* args[] = {&a};
  if (exclusive) {
    // Ordinary dispatch on the caller's queue: all G workgroups fit at once
    // (checked above), so on a device running nothing else they are all
    // resident.  Saves the hand-off to and from the runtime's cooperative
    // queue (about 20 us per solve).
    e = hipLaunchKernel((const void*)kern, dim3(a.G), dim3(NT), args, (unsigned)lds, st);
    if (e != hipSuccess) return fail_hip(e, "grid pcg launch");
  } else {
    e = hipLaunchCooperativeKernel((const void*)kern, dim3(a.G), dim3(NT), args,
                                   (unsigned)lds, st);
    if (e == hipErrorCooperativeLaunchTooLarge)
      return fail(GLASS_ECOOP, "grid pcg: cooperative launch too large");
    if (e != hipSuccess) return fail_hip(e, "grid pcg cooperative launch");
  }
  epoch_commit(dev.device, area, keep, a.max_iters, ep);
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
                    bool exclusive, bool single, void* area, size_t area_bytes, bool keep,
                    hipStream_t st) {
  if constexpr (kGridResidentFits<T>(SS))
    return launch_grid_typed<T, SS, true>(a, NT, lds, dev, exclusive, single, area, area_bytes,
                                          keep, st);
  return fail(GLASS_EUNSUPPORTED, "grid pcg: internal plan error");
}

// workspace == nullptr: the exchange area is this device's static scratch
// (glass_pcg_grid_noalloc), laid out for the grid actually launched.
template <typename T>
int launch_grid(T* x, const T* S, const T* P, const T* b, int ss, int kp,
                int max_iters, double rel_tol, double abs_tol, int* iters,
                int* status, T* rho, void* workspace, size_t ws_bytes,
                bool exclusive, bool single, bool keep, hipStream_t st) {
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  if (!dev.cooperative)
    return fail(GLASS_ECOOP, "device does not support cooperative launches");
  const bool own_scratch = workspace == nullptr;
  if (!own_scratch && ws_bytes < layout(ss, kp, sizeof(T)).total)
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
  const int NW = NT / 64;
  const size_t loc_len = (size_t)(nb_max + 4) * ss;
  const size_t lds = (2 * loc_len + 8 * (size_t)ss + (size_t)kDotValues * (NW + 1)) * sizeof(T);
  if (lds > dev.max_lds_per_block)
    return fail(GLASS_EUNSUPPORTED, "grid pcg: partition does not fit in LDS");
  WorkspaceLayout wl = layout(ss, kp, sizeof(T));
  if (own_scratch) {
    wl = layout_for((size_t)G, ss, sizeof(T));
    if (wl.total > kNoAllocScratchBytes)
      return fail(GLASS_EUNSUPPORTED,
                  "grid pcg (no-alloc): " + std::to_string(G) + " workgroups need " +
                      std::to_string(wl.total) + " bytes of exchange area, more than the " +
                      std::to_string(kNoAllocScratchBytes) + " bytes of static scratch");
    if (int rc = scratch_address(dev.device, &workspace)) return rc;
    ws_bytes = kNoAllocScratchBytes;
    keep = true;  // only these solves ever write the library's own scratch
  }

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
  a.flags = reinterpret_cast<unsigned int*>(ws + wl.flags);
  a.part = reinterpret_cast<u64*>(ws + wl.part);
  a.edges = reinterpret_cast<u64*>(ws + wl.edges);
  a.G = G;
  a.nb_max = nb_max;
  a.wide = aligned(S, 16) && aligned(P, 16);
  a.spin_limit = kSpinLimit;
  if (const char* sl = tuning_getenv("GLASS_AMD_GRID_SPIN_LIMIT"); sl && *sl) {
    char* end = nullptr;
    const unsigned long v = std::strtoul(sl, &end, 10);
    if (end != sl && *end == '\0' && v <= kSpinLimit) a.spin_limit = (unsigned)v;
  }
  if (res) {
    switch (ss) {
      case 6: return launch_grid_res<T, 6>(a, NT, lds, dev, exclusive, single, workspace, ws_bytes,
                                           keep, st);
      case 12: return launch_grid_res<T, 12>(a, NT, lds, dev, exclusive, single, workspace,
                                             ws_bytes, keep, st);
      case 14: return launch_grid_res<T, 14>(a, NT, lds, dev, exclusive, single, workspace,
                                             ws_bytes, keep, st);
      default: return launch_grid_res<T, 21>(a, NT, lds, dev, exclusive, single, workspace,
                                             ws_bytes, keep, st);
    }
  }
  return launch_grid_typed<T, 0, false>(a, NT, lds, dev, exclusive, single, workspace, ws_bytes,
                                        keep, st);
}

}  // namespace

size_t grid_workspace_bytes(int ss, int kp, glass_dtype dt) {
  return layout(ss, kp, dt == GLASS_F32 ? sizeof(float) : sizeof(double)).total;
}

int launch_pcg_grid(glass_dtype dt, void* x, const void* S, const void* Pinv,
                    const void* b, int ss, int kp, int max_iters,
                    double rel_tol, double abs_tol, int* iters, int* status,
                    void* rho, void* workspace, size_t workspace_bytes,
                    bool exclusive, bool single, bool keep, hipStream_t stream) {
  if (dt == GLASS_F32)
    return launch_grid<float>((float*)x, (const float*)S, (const float*)Pinv,
                              (const float*)b, ss, kp, max_iters, rel_tol,
                              abs_tol, iters, status, (float*)rho, workspace,
                              workspace_bytes, exclusive, single, keep, stream);
  return launch_grid<double>((double*)x, (const double*)S, (const double*)Pinv,
                             (const double*)b, ss, kp, max_iters, rel_tol,
                             abs_tol, iters, status, (double*)rho, workspace,
                             workspace_bytes, exclusive, single, keep, stream);
}

}  // namespace glass
