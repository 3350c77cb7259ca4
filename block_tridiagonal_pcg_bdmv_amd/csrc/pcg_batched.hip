// Batched preconditioned conjugate gradient, one problem per workgroup
// (GLASS user guide, page "Block-tridiagonal Solves", section
// "Solve -- glass::pcg"; the matvec windows follow sections "The [L|D|R]
// block-tridiagonal layout" and "The padded vector layout").
//
// Steps per problem (standard PCG; the page fixes the z = p = Pinv r start,
// rho = r^T z and the stopping rule |rho| < abs_tol + rel_tol |rho_init|):
//   r = b - S x; z = Pinv r; p = z; rho = r^T z; rho_init = |rho|
//   loop: Sp = S p; alpha = rho / p^T Sp; x += alpha p; r -= alpha Sp;
//         z = Pinv r; rho' = r^T z; stop if |rho'| < thresh;
//         p = z + (rho'/rho) p; rho = rho'
//
// Mapping on gfx950 (wave64):
// * rows are dealt to waves in 64-row chunks: chunk c goes to wave c % NW and
//   lane l of that wave owns row 64c + l; a lane owns RPT rows.  Its entries of
//   x, r, p (and the transient z, S p) live in registers.
// * only p and r must be seen by other lanes (the 3*ss matvec window), so
//   they are the two padded vectors kept in LDS; the page's other work
//   vectors stay in registers.  Where S (or both matrices) stays on chip,
//   each block of ss entries takes a whole number of 16-byte vectors in LDS,
//   so a window is read with 16-byte loads.
// * dots: each 64-row chunk's products -> wave64 DPP tree -> one LDS slot per
//   chunk -> every thread adds the slots in chunk order.  alpha, beta and the
//   stopping decision are therefore computed identically (same bits) by every
//   thread and need no broadcast, and the whole solve is bit-identical for
//   every placement (number of waves, rows per lane, resident or streamed).
//   Two slot arrays alternate so one barrier per dot suffices.
// * matrices: RESIDENT -- each lane holds its S row and Pinv row in VGPRs,
//   loaded once: straight from memory with every load of both rows in
//   flight (the widest loads the row alignment allows), or (RESD) through
//   the wave's LDS stage by coalesced direct loads -- the Pinv rows, and the
//   S rows first when rows are 128 bytes or longer;
//   STREAMED -- every matvec re-stages the wave's 64-row chunk of S or
//   Pinv HBM/L2 -> LDS (coalesced 16-byte loads) and each lane multiplies its
//   row from there.  With PREFETCH, the wave's next chunk (two with
//   GLASS_AMD_RING_DEPTH=2) in the fixed sequence (chunks of S, then of
//   Pinv, then of S, ...) is loaded into registers ahead of use, so it stays
//   in flight across the multiply, the dots and the workgroup barriers
//   (matrix loads never depend on the vectors);
//   S RESIDENT (HYBRID) -- when S and Pinv rows do not fit the registers
//   together: each lane holds its S rows in VGPRs for the whole solve, and
//   Pinv goes memory -> LDS with direct buffer -> LDS loads, which hold no
//   registers in flight.  A general Pinv streams through a per-wave stage a
//   chunk at a time, each pass walking the wave's chunks in the opposite
//   direction to the pass before, so a pass after the first starts with the
//   chunk the previous one left in the stage and does not load it again
//   (some chunks pinned on chip for the whole solve: in LDS left over after
//   the stages, or in the S registers of waves without a last chunk); a
//   block-Jacobi Pinv's D blocks are loaded whole into LDS once.
// Barriers per iteration: 4 (p^T Sp, r publish, r^T z, p publish).
//
// RESIDENT with a block-diagonal Pinv (the caller asserts its L and R blocks
// are zero): each lane holds only the D part of its Pinv row and multiplies
// it with its own block-row of r.  The skipped terms are exact zeros that the
// general contraction adds after and before the D terms, so the result has
// the same value; fewer registers let more workgroups share a CU.  STREAMED
// with PREFETCH and a block-diagonal Pinv: a Pinv chunk's 16-byte vectors
// that touch no row's D block are given an offset past the buffer's end, so
// they read zeros and are not fetched (about 2/5 of the vectors remain at
// ss=21).
//
// Pinv as packed D blocks ([kp*ss][ss] per problem, the same block-Jacobi
// preconditioner stored without its zero blocks): resident lanes load their
// ss values from row*ss, and streamed chunks are 64 rows of ss values,
// multiplied with the middle third of the window.  The terms and their order
// are those of the D-only rows above, so the results are the same; every
// byte fetched is a D byte.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

// Chunks a wave keeps in flight in the prefetching placement (1 or 2).
#ifndef GLASS_AMD_RING_DEPTH
#define GLASS_AMD_RING_DEPTH 1
#endif

// S rows of the streamed S-resident placement: 1 = each wave's chunks are
// loaded coalesced into its LDS stage by direct loads, then copied into
// registers; 0 = loaded per lane straight into registers.
#ifndef GLASS_AMD_HYB_S_VIA_LDS
#define GLASS_AMD_HYB_S_VIA_LDS 1
#endif

namespace glass {
namespace {

constexpr int kRingDepth = GLASS_AMD_RING_DEPTH;
constexpr bool kSViaLds = GLASS_AMD_HYB_S_VIA_LDS != 0;
static_assert(kRingDepth == 1 || kRingDepth == 2, "ring depth must be 1 or 2");

template <typename T>
struct PcgArgs {
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
  int vec;          // 16-byte staging allowed (alignment checked on the host)
  int stage_elems;  // per-wave LDS stage, elements
  int npin;         // HYBRID streaming: waves below npin keep their last Pinv
                    // chunk pinned in LDS (loaded once)
  int regpin;       // HYBRID streaming: a wave without a last chunk keeps its
                    // chunk 0 of Pinv in the registers that leaves free
  int ppacked;      // Pinv is packed D blocks, [kp*ss][ss] per problem (read
                    // by kStream; the other modes fix it at compile time)
  unsigned lds_bytes;  // dynamic LDS of the launch (debug fill)
  int resd_s_stage;    // RESD: S rows also arrive through the stage, before Pinv's
                       // (coalesced; one exposed round trip)
  int preg_stage;      // HYBS: preg waves' Pinv chunk 0 arrives through the stage
                       // after their S chunks (coalesced), not row by row
};

// Block stride of the padded vectors in LDS: ss rounded up to whole 16-byte
// vectors, so every window starts 16-byte aligned and its reads can be
// 16-byte LDS loads (twice the delivery rate of 4- and 8-byte ones).  The
// tail of each block is never read.  The placements that hold S (or both
// matrices) on chip use it; the streamed ones keep blocks of ss (they
// measured no faster padded, and the plain streamed placement, the
// fallback for the largest problems, needs the least LDS).
template <typename T>
__host__ __device__ constexpr int vec_block(int ss, bool padded = true) {
  return padded ? (ss + (int)(16 / sizeof(T)) - 1) / (int)(16 / sizeof(T)) * (int)(16 / sizeof(T))
                : ss;
}

// Placements of the matrices (see the header).
enum Mode {
  kResident = 0,
  kStreamPrefetch = 1,
  kStream = 2,
  kResidentPD = 3,        // resident, Pinv's D blocks only
  kStreamPrefetchPD = 4,  // streamed with prefetch, Pinv vectors touching D only
  kStreamPrefetchPDP = 5,  // streamed with prefetch, Pinv as packed D blocks
  kResidentPDP = 6,        // resident, Pinv as packed D blocks
  kHybrid = 7,             // S resident, Pinv streamed by direct loads into LDS
  kHybridPDP = 8,          // S resident, Pinv's packed D blocks held whole in LDS
  kHybridPD = 9,           // S resident, D parts of the [L|D|R] Pinv gathered into LDS
  kResidentDma = 10,       // resident; Pinv rows arrive through the wave's LDS stage
};

// Workgroup size bound: 8 waves (so a lane may use up to 256 VGPRs) for the
// prefetching placement (two chunk buffers per lane) and for 3-4 rows per
// lane; 16 waves otherwise (rows beyond 4096 need them, at the cost of
// spills).
constexpr int max_threads_for(int rpt, int mode) {
  const bool resident = mode == kResident || mode == kResidentPD || mode == kResidentPDP ||
                        mode == kResidentDma;
  return (mode == kStreamPrefetch || mode == kStreamPrefetchPD || mode == kStreamPrefetchPDP ||
          mode == kHybrid || mode == kHybridPDP || mode == kHybridPD || rpt == 3 || rpt == 4 ||
          (resident && rpt > 1))
             ? 512
             : 1024;
}

template <typename T, int SS, int RPT, int MODE>
__global__ void __launch_bounds__(max_threads_for(RPT, MODE))
pcg_batched_kernel(PcgArgs<T> a) {
  constexpr bool RES = MODE == kResident || MODE == kResidentPD || MODE == kResidentPDP ||
                       MODE == kResidentDma;
  // RESD: resident rows, with each wave's 64 Pinv rows brought into its LDS
  // stage by coalesced direct loads (no registers in flight) while the S
  // rows load straight into registers; each lane then copies its Pinv row.
  constexpr bool RESD = MODE == kResidentDma;
  constexpr bool PD = MODE == kResidentPD || MODE == kResidentPDP;  // Pinv rows: D part only
  constexpr bool PFM =
      MODE == kStreamPrefetch || MODE == kStreamPrefetchPD || MODE == kStreamPrefetchPDP;
  // HYBRID: S rows resident in registers; Pinv chunks streamed into the
  // wave's LDS stage by direct buffer -> LDS loads (HYBS), or Pinv's D blocks
  // loaded whole into LDS once the same way (HYBP): copied when Pinv comes as
  // packed D blocks, gathered from the [L|D|R] rows under the block-diagonal
  // hint.
  constexpr bool HYBS = MODE == kHybrid;
  constexpr bool HYBP = MODE == kHybridPDP || MODE == kHybridPD;
  constexpr bool HYB = HYBS || HYBP;
  constexpr bool SRES = RES || HYB;  // S rows held in registers
  // Pinv chunks of packed D blocks in the prefetch ring (compile time, so the
  // ring keeps one load pattern per position).
  constexpr bool PFP = MODE == kStreamPrefetchPDP;
  constexpr int WC = SS > 0 ? 3 * SS : 1;  // compile-time width
  const int ss = SS > 0 ? SS : a.ss;
  const int W = 3 * ss;
  const int kp = a.kp;
  const int n = kp * ss;
  // p and r in LDS as kp + 2 blocks of ssp elements (a zero block at each
  // end, ss entries used per block).
  constexpr bool PADV = RES || HYBP || HYBS;
  constexpr int SSP = SS > 0 ? vec_block<T>(SS, PADV) : 0;
  const int ssp = SS > 0 ? SSP : vec_block<T>(ss, PADV);
  const int pad_len = (kp + 2) * ssp;
  const int NT = blockDim.x;
  const int NW = NT >> 6;
  const int tid = threadIdx.x;
  // The wave index is uniform within a wave; saying so keeps everything
  // derived from it (chunk rows, buffer resources) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const long long prob = blockIdx.x;
  const long long mstride = (long long)n * W;
  // Pinv as packed D blocks: fixed by the mode, except for plain staging.
  const bool packed = MODE == kResidentPDP || MODE == kStreamPrefetchPDP || MODE == kHybridPDP ||
                      (MODE == kStream && a.ppacked != 0);
  const T* __restrict__ gS = a.S + prob * mstride;
  const T* __restrict__ gP = a.P + prob * (packed ? (long long)n * ss : mstride);
  const bool vec = a.vec != 0;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_debug_fill(smem_raw, a.lds_bytes);
  T* p_pad = reinterpret_cast<T*>(smem_raw);
  T* r_pad = p_pad + pad_len;
  const int nchunks = (n + 63) / 64;
  T* slotA = r_pad + pad_len;  // [nchunks] per-chunk dot partials
  T* slotB = slotA + nchunks;
  const size_t head = ((size_t)(2 * pad_len + 2 * nchunks) * sizeof(T) + 15) & ~(size_t)15;
  // Every stage holds a whole number of 64-row blocks (the host sizes it as
  // 64 rows of a fixed width), so every stage starts as aligned as the head.
  __builtin_assume(a.stage_elems % 64 == 0);
  T* stage = reinterpret_cast<T*>(smem_raw + head) + (size_t)wave * a.stage_elems;
  // HYBS: a wave below a.npin holds its last chunk (k = RPT-1) of Pinv in a
  // pinned slot after the NW stages, loaded once; only its other chunks
  // stream.  Host: RPT >= 2 and the slots fit in LDS.
  const bool pin_last = HYBS && wave < a.npin;  // wave-uniform
  T* pinned = reinterpret_cast<T*>(smem_raw + head) + (size_t)(NW + wave) * a.stage_elems;
  // HYBS: a wave with chunk 0 but no chunk at k = RPT-1 keeps the Pinv rows
  // of its chunk 0 in the S registers that position leaves unused (loaded
  // once); only its chunks in between stream.
  const bool preg = HYBS && a.regpin != 0 && RPT >= 2 && (wave + (RPT - 1) * NW) * 64 >= n &&
                    wave * 64 < n;  // wave-uniform
  // Positions k of the wave's chunk sequence that do not stream through the
  // stage: the LDS-pinned last chunk, and for preg waves chunk 0 and the
  // positions past the wave's chunks.
  auto no_stream = [&](int k) {
    return (pin_last && k == RPT - 1) || (preg && (k == 0 || (wave + k * NW) * 64 >= n));
  };
  // HYBS: positions whose chunk exists and goes through the stage.
  auto streams = [&](int k) { return !no_stream(k) && (wave + k * NW) * 64 < n; };
  // HYBP: the problem's packed Pinv D blocks, [n][ss], after the head.
  T* pinv_lds = reinterpret_cast<T*>(smem_raw + head);

  // Row bookkeeping.
  int row[RPT], wstart[RPT], vix[RPT];
  bool valid[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    row[k] = (wave + k * NW) * 64 + lane;
    valid[k] = row[k] < n;
    const int br = valid[k] ? row[k] / ss : 0;
    wstart[k] = br * ssp;                         // window start in a padded vector
    vix[k] = (br + 1) * ssp + (row[k] - br * ss);  // the row's own entry
    // Blocks of whole 16-byte vectors: every window starts 16-byte aligned
    // (said here because the compiler rewrites br * ssp as row - row % ss).
    if constexpr (SS > 0 && (SSP * sizeof(T)) % 16 == 0)
      __builtin_assume((wstart[k] & (int)(16 / sizeof(T) - 1)) == 0);
  }
  // Window entry c (0 <= c < 3*ss) of a padded vector window w: block c / ss,
  // entry c % ss.  The window start is 16-byte aligned.
  auto win = [&](const T* __restrict__ w, int c) -> T {
    const T* __restrict__ wa = w;
    if constexpr (PADV) wa = static_cast<const T*>(__builtin_assume_aligned(w, 16));
    return SS > 0 ? wa[(c / SS) * SSP + c % SS] : wa[(c / ss) * ssp + c % ss];
  };

  // Chunk k of this wave: rows [r0, r0 + nrows) of a matrix, which are one
  // contiguous range of count = nrows * W elements.
  auto chunk_r0 = [&](int k) { return (wave + k * NW) * 64; };

  // Buffer-load the wave's chunk k of gM as 16-byte vectors in the coalesced
  // order (lane l gets vectors l, l+64, ...).  The resource spans exactly the
  // chunk's bytes and the hardware range-checks raw buffer loads per dword:
  // dwords past the end read as zeros without touching memory, so a chunk
  // that ends inside a vector still arrives whole, no lane branches, and one
  // offset register serves every load.  A chunk this wave does not have
  // (r0 >= n) becomes an empty resource: the loads return zeros.
  constexpr int NV = (WC * (int)sizeof(T) + 15) / 16;  // vectors per lane
  // A chunk of packed D blocks (rows of ss elements) is NVD vectors per lane.
  constexpr int NVD = ((SS > 0 ? SS : 1) * (int)sizeof(T) + 15) / 16;
  auto load_chunk = [&](vec16_t (&buf)[NV], const T* __restrict__ gM, int k, bool dpart,
                        bool dpacked) {
    const int r0 = chunk_r0(k);
    const bool has = r0 < n;
    const int rw = dpacked ? ss : W;  // elements per row in gM
    const int nbytes = has ? min(64, n - r0) * rw * (int)sizeof(T) : 0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(has ? gM + (long long)r0 * rw : gM, nbytes);
    if (dpacked) {
#pragma unroll
      for (int u = 0; u < NVD; ++u) buf[u] = buffer_load16(rs, (lane + u * kWave) * 16);
      return;
    }
    constexpr int RB = WC * (int)sizeof(T);                  // row bytes
    constexpr int D0 = (SS > 0 ? SS : 1) * (int)sizeof(T);  // D block bytes [D0, 2*D0)
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      int off = (lane + u * kWave) * 16;
      if (dpart) {
        // Does [off, off+16) touch the D block of its row or of the next?
        const int q = off / RB, in = off - q * RB;
        const bool touch = (in < 2 * D0 && in + 16 > D0) || (in + 16 - RB > D0);
        off = touch ? off : 0x7ffffff0;  // past the end: zeros, no fetch
      }
      buf[u] = buffer_load16(rs, off);
    }
  };
  // Write a loaded chunk into the wave's LDS stage (same layout as in HBM; the
  // stage holds NV*64 vectors, so every store is in bounds).
  auto stage_chunk = [&](const vec16_t (&buf)[NV], bool dpacked) {
    vec16_t* __restrict__ d4 = reinterpret_cast<vec16_t*>(stage);
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (!dpacked || u < NVD) d4[lane + u * kWave] = buf[u];
  };

  // RESIDENT: each lane's S and Pinv rows in registers for the whole solve,
  // loaded straight from HBM with every load of both rows in flight.
  constexpr int WCP = PD ? (SS > 0 ? SS : 1) : WC;  // Pinv row width held
  T mS[SRES ? RPT : 1][WC], mP[RES ? RPT : 1][WCP];
  if constexpr (SRES) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
#pragma unroll
      for (int c = 0; c < WC; ++c) mS[k][c] = T(0);
      if constexpr (RES) {
#pragma unroll
        for (int c = 0; c < WCP; ++c) mP[k][c] = T(0);
      }
      if (valid[k] && !(HYBS && kSViaLds) && !(RESD && a.resd_s_stage)) {
        const long long off = (long long)row[k] * WC;
        // The D part starts ss elements into the row: at (3*row + 1) times
        // its own byte size, so the widths load_row_regs picks stay aligned.
        // Packed D blocks: the row's ss values start at row * ss.
        const long long offP =
            MODE == kResidentPDP ? (long long)row[k] * SS : off + (PD ? SS : 0);
        if (vec) {
          load_row_regs<T, WC, true>(mS[k], gS + off);
          if constexpr (RES && !RESD) load_row_regs<T, WCP, true>(mP[k], gP + offP);
        } else {
          load_row_regs<T, WC, false>(mS[k], gS + off);
          if constexpr (RES && !RESD) load_row_regs<T, WCP, false>(mP[k], gP + offP);
        }
      }
    }
  }
  if constexpr (HYBS) {
    // preg: chunk 0's Pinv rows into the registers of the absent last chunk.
    if (preg && valid[0] && !(kSViaLds && a.preg_stage)) {
      if (vec) load_row_regs<T, WC, true>(mS[RPT - 1], gP + (long long)row[0] * WC);
      else load_row_regs<T, WC, false>(mS[RPT - 1], gP + (long long)row[0] * WC);
    }
  }

  // HYBRID: chunk k of this wave's rows of a matrix (Pinv, or S once at the
  // start), loaded straight into LDS at dst in the coalesced order (lane l's
  // 16-byte vectors l, l+64, ... land at the same offsets as in memory, so
  // dst has the chunk's layout).  The resource spans exactly the chunk;
  // vectors past its end, or every vector of a chunk the wave does not have,
  // write zeros without a fetch.  The loads use no registers once issued, so
  // the next Pinv chunk is in flight while the wave multiplies, reduces and
  // waits at barriers.
  //
  // Matrices aligned to the element size only: the chunk is loaded from the
  // 16-byte boundary at or below its first byte (the same 16-byte granule of
  // the caller's allocation), so it lands `shift` bytes into dst, and readers
  // add the shift (stage_shift).  64 rows of 3ss elements are a multiple of
  // 16 bytes, so the shift is the same for every chunk of one matrix of one
  // problem; the host uses this only where the stage has the spare bytes.
  auto dma_rows_to = [&](const T* __restrict__ gM, int k, T* dst) {
    if constexpr (HYBS) {
      const int r0 = chunk_r0(k);
      const bool has = r0 < n;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(gM + (long long)r0 * W);
      const int shift = (int)(reinterpret_cast<uintptr_t>(src) & 15u);
      const int nbytes = has ? min(64, n - r0) * W * (int)sizeof(T) + shift : 0;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(has ? src - shift : src, nbytes);
      unsigned char* st = reinterpret_cast<unsigned char*>(dst);
      // The lane's byte offset, made opaque here so that the offsets of the
      // NV loads are formed at each call instead of being kept in NV
      // registers for the whole solve.
      int vbase = lane * 16;
      asm volatile("" : "+v"(vbase));
      // S is read once: in fp64 its loads are non-temporal (cache-policy
      // bit 1), which measured 414 -> 401 us on the fp64 ss=14 solve; in
      // fp32 the same slowed the ss=21 solve (440 -> 466 us).
      if (sizeof(T) == 8 && gM == gS) {
#pragma unroll
        for (int u = 0; u < NV; ++u)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(st + u * kWave * 16), 16,
              vbase + u * kWave * 16, 0, 0, 2);
      } else {
#pragma unroll
        for (int u = 0; u < NV; ++u)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(st + u * kWave * 16), 16,
              vbase + u * kWave * 16, 0, 0, 0);
      }
    }
  };
  auto dma_chunk_to = [&](int k, T* dst) { dma_rows_to(gP, k, dst); };
  // Where a matrix's chunk starts inside the stage it was loaded into.
  auto stage_shift = [&](const T* __restrict__ gM, const T* buf) {
    return reinterpret_cast<const T*>(reinterpret_cast<const unsigned char*>(buf) +
                                      (reinterpret_cast<uintptr_t>(gM) & 15u));
  };
  auto dma_chunk = [&](int k) { dma_chunk_to(k, stage); };

  // HYBP: every wave loads pieces q = wave, wave + NW, ... of the problem's
  // D blocks into pinv_lds, laid out [n][ss].  Packed D blocks are one
  // contiguous range, copied in 1 KB pieces (the range check zero-fills the
  // last piece past the data).  Under the block-diagonal hint each lane
  // gathers one 4-byte word of a D block from its [L|D|R] row (256-byte
  // pieces; words past the D blocks read zeros).  Each wave waits for its
  // own pieces before the barrier that precedes the first Pinv matvec.
  auto dma_pinv_whole = [&]() {
    if constexpr (MODE == kHybridPD) {
      constexpr int DPE = (int)sizeof(T) / 4;  // 4-byte words per element
      const int nwords = n * SS * DPE;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(gP, n * W * (int)sizeof(T));
      const int npieces = (nwords + kWave - 1) / kWave;
      unsigned char* base = reinterpret_cast<unsigned char*>(pinv_lds);
      for (int q = wave; q < npieces; q += NW) {
        const int d = q * kWave + lane;  // word of the [n][ss] D layout
        const int e = d / DPE, r = e / SS, c = e - r * SS;
        const int off = d < nwords ? (r * 3 * SS + SS + c) * (int)sizeof(T) + (d - e * DPE) * 4
                                   : 0x7ffffff0;  // past the end: zero
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(base + q * kWave * 4), 4, off, 0, 0,
            0);
      }
    } else if constexpr (HYBP) {
      const int nbytes = n * ss * (int)sizeof(T);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(gP, nbytes);
      const int npieces = (nbytes + kWave * 16 - 1) / (kWave * 16);
      unsigned char* base = reinterpret_cast<unsigned char*>(pinv_lds);
      for (int q = wave; q < npieces; q += NW)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(base + q * kWave * 16), 16,
            q * kWave * 16 + lane * 16, 0, 0, 0);
    }
  };

  // Workgroup barrier.  HYBRID orders LDS only: a release fence would also
  // wait for the wave's direct loads in flight, which only the wave itself
  // reads (after its own vmcnt wait), and global memory is not shared
  // between the waves before the final stores.
  auto block_sync = [&]() {
    if constexpr (HYB || RESD) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
  };

  // PREFETCH: a two-deep ring of chunk buffers.  The wave walks the fixed
  // sequence of positions pos = m*RPT + k (m = 0 for S, 1 for Pinv; matvecs
  // alternate S, Pinv, S, ...), and position pos lives in buffer pos % 2.
  // After staging position pos it loads position pos + 2 (mod 2*RPT) into
  // the buffer it just emptied, so two chunks are in flight while the wave
  // multiplies, reduces and waits at barriers.  Every position is loaded
  // (empty for a chunk the wave does not have), so the loads form one
  // unbranched in-order stream and each staging waits only for its own
  // buffer.
  vec16_t pf0[PFM ? NV : 1], pf1[PFM ? NV : 1];
  auto ring_load = [&](int pos) {
    if constexpr (PFM) {
      const int m = pos / RPT, k = pos % RPT;
      const T* gM = m == 0 ? gS : gP;
      const bool dpart = MODE == kStreamPrefetchPD && m == 1;
      const bool dpacked = PFP && m == 1;
      if constexpr (kRingDepth == 1) {
        load_chunk(pf0, gM, k, dpart, dpacked);
      } else {
        if (pos % 2 == 0) load_chunk(pf0, gM, k, dpart, dpacked);
        else load_chunk(pf1, gM, k, dpart, dpacked);
      }
    }
  };

  // out[k] = (M * vpad)[row k]: one lane, one row, serial 3*ss contraction.
  // MI selects the matrix: 0 = S, 1 = Pinv.  REV walks the wave's chunk
  // positions from the last to the first (each row's result does not depend
  // on the order; HYBS uses it to start a pass with the chunk the previous
  // pass left in the stage).
  auto matvec = [&](auto mi_tag, T (&out)[RPT], auto& mreg, const T* __restrict__ vpad,
                    auto rev_tag) {
    constexpr int MI = decltype(mi_tag)::value;
    constexpr bool REV = decltype(rev_tag)::value;
    const T* __restrict__ gM = MI == 0 ? gS : gP;
    // Streamed Pinv as packed D blocks: rows of ss values, multiplied with
    // the middle third of the window (the terms and order of a D-only row).
    // Prefetching placements know it at compile time.
    const bool mpacked = MI == 1 && (PFM ? PFP : packed);
    constexpr bool REG = MI == 0 ? SRES : RES;  // this matrix's rows in registers
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int k = REV ? RPT - 1 - j : j;
      T acc = T(0);
      if constexpr (REG) {
        if (valid[k]) {
          const T* __restrict__ w = vpad + wstart[k];
          if constexpr (PD && MI == 1) {
#pragma unroll
            for (int c = 0; c < WCP; ++c) acc = fma(mreg[k][c], win(w, SS + c), acc);
          } else {
#pragma unroll
            for (int c = 0; c < WC; ++c) acc = fma(mreg[k][c], win(w, c), acc);
          }
        }
      } else if constexpr (HYBS) {
        // Pinv chunk k is pinned in LDS, held in registers (preg waves'
        // chunk 0), or in (or on its way to) the stage.  For the stage: wait
        // for this wave's direct loads, multiply, and once every stage read
        // has returned, load the next streamed chunk of this matvec (in its
        // walking order) into it.  Passes alternate direction, so each pass
        // after the first starts with the chunk the previous one left in
        // the stage: it is not loaded again, and no load is in flight
        // between passes (a solve that stops fetches nothing more).
        const bool from_pin = pin_last && k == RPT - 1;  // wave-uniform
        const bool from_reg = preg && k == 0;             // wave-uniform
        const bool streamed = streams(k);
        if (streamed) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (chunk_r0(k) < n) {  // wave-uniform
          if (valid[k]) {
            const T* __restrict__ w = vpad + wstart[k];
            if (from_reg) {
#pragma unroll
              for (int c = 0; c < WC; ++c) acc = fma(mS[RPT - 1][c], win(w, c), acc);
            } else {
              const T* __restrict__ m = stage_shift(gP, from_pin ? pinned : stage) + lane * W;
#pragma unroll 3
              for (int c0 = 0; c0 < 3 * SS; c0 += SS) {
#pragma unroll
                for (int c = c0; c < c0 + SS; ++c) acc = fma(m[c], win(w, c), acc);
              }
            }
          }
          if (streamed) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        if (streamed) {
          int next = -1;  // the next streamed position of this matvec
          if constexpr (REV) {
            for (int q = k - 1; q >= 0 && next < 0; --q)
              if (streams(q)) next = q;
          } else {
            for (int q = k + 1; q < RPT && next < 0; ++q)
              if (streams(q)) next = q;
          }
          if (next >= 0) dma_chunk(next);
        }
      } else if constexpr (HYBP) {
        // The row's ss values of its D block, times the middle third of the
        // window (the terms and order of a D-only row).
        if (valid[k]) {
          const T* __restrict__ m = pinv_lds + row[k] * SS;
          const T* __restrict__ w = vpad + wstart[k];
#pragma unroll
          for (int c = 0; c < SS; ++c) acc = fma(m[c], win(w, SS + c), acc);
        }
      } else {
        const int r0 = chunk_r0(k);
        if constexpr (PFM) {
          constexpr int pos = MI * RPT;  // + k, below
          if (r0 < n) {  // wave-uniform
            if constexpr (kRingDepth == 1) {
              stage_chunk(pf0, mpacked);
            } else {
              if ((pos + k) % 2 == 0) stage_chunk(pf0, mpacked);
              else stage_chunk(pf1, mpacked);
            }
          }
          // Keep the next loads after these LDS stores, so the emptied
          // buffer's registers are reused (the compiler would otherwise
          // hoist the loads and hold an extra chunk).
          asm volatile("" ::: "memory");
          // Position pos + depth goes into this position's buffer, whether
          // or not this position had a chunk for this wave.
          ring_load((pos + k + kRingDepth) % (2 * RPT));
        }
        if (r0 < n) {  // wave-uniform
          if constexpr (!PFM) {
            const int nrows = min(64, n - r0);
            const int rw = mpacked ? ss : W;
            copy_to_lds<false>(stage, gM + (long long)r0 * rw, nrows * rw, lane, kWave, vec);
          }
          wave_lds_sync();
          if (valid[k] && mpacked) {
            const T* __restrict__ m = stage + lane * ss;
            const T* __restrict__ w = vpad + wstart[k];
            if constexpr (SS > 0) {
#pragma unroll
              for (int c = 0; c < SS; ++c) acc = fma(m[c], win(w, SS + c), acc);
            } else {
              const T* __restrict__ wd = w + ssp;
              for (int c = 0; c < ss; ++c) acc = fma(m[c], wd[c], acc);
            }
          } else if (valid[k]) {
            const T* __restrict__ m = stage + lane * W;
            const T* __restrict__ w = vpad + wstart[k];
            if constexpr (SS > 0) {
              // Partial unroll: bounds the LDS reads in flight (registers).
#pragma unroll 3
              for (int c0 = 0; c0 < 3 * SS; c0 += SS) {
#pragma unroll
                for (int c = c0; c < c0 + SS; ++c) acc = fma(m[c], win(w, c), acc);
              }
            } else {
              // Three blocks of ss entries, in the order of the row.
              for (int b3 = 0; b3 < 3; ++b3)
                for (int c = 0; c < ss; ++c)
                  acc = fma(m[b3 * ss + c], w[b3 * ssp + c], acc);
            }
          }
          wave_lds_sync();
        }
      }
      out[k] = acc;
    }
  };
  using MatS = std::integral_constant<int, 0>;
  using MatP = std::integral_constant<int, 1>;
  using Fwd = std::integral_constant<bool, false>;
  using Rev = std::integral_constant<bool, HYBS>;  // reverse order only where it pays

  // Dot product of two row-distributed vectors, independent of the launch
  // shape: each 64-row chunk's products go through the fixed wave64 tree
  // into its own LDS slot, and every thread adds the slots in chunk order.
  // The result has the same bits in every thread and for every placement
  // (waves, rows per lane, resident or streamed).  One __syncthreads();
  // the two slot arrays alternate so a read of one use never meets a write
  // of the next.
  auto chunk_dot = [&](const T (&u)[RPT], const T (&v)[RPT], T* slots) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      if (chunk_r0(k) < n) {  // wave-uniform
        const T c = wave_sum(mul_unfused(u[k], v[k]));
        if (lane == 0) slots[wave + k * NW] = c;
      }
    }
    block_sync();
    // Resident placements: all slots in one LDS round trip, added from the
    // lanes in order.  The others keep the slot-by-slot loop, which measured
    // faster there: the S-resident kernels hold 3*ss S values per lane, and
    // the lane form's extra live values left their stage matvec fewer
    // registers for LDS reads in flight (1-4 % slower).  Both add the same
    // values in the same order, so the bits agree.
    if constexpr (RES) {
      return sum_slots_in_order(slots, nchunks);
    } else {
      T s = slots[0];
      for (int c = 1; c < nchunks; ++c) s = s + slots[c];
      return s;
    }
  };

  // Initial state: p_pad temporarily holds x0 (the vector S multiplies).
  // x0 and b are loaded before the first matrix chunks so that waiting for
  // them does not wait for the chunks too (loads complete in order).
  T xr[RPT], rr[RPT], pr[RPT], tmp[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    xr[k] = T(0);
    tmp[k] = T(0);
    if (valid[k]) {
      xr[k] = a.x[prob * n + row[k]];
      tmp[k] = a.b[prob * n + row[k]];
    }
  }
  if constexpr (PFM) {
    ring_load(0);
    if (kRingDepth == 2) ring_load(1 % (2 * RPT));
  }
  if constexpr (RESD) {
    // This wave's Pinv rows (one chunk: RPT == 1) into its stage, issued
    // after x0 and b so that waiting for those does not wait for them.  The
    // stage holds exactly the chunk; lanes past its last 16-byte vector are
    // masked off.  With resd_s_stage the wave's S rows come the same way
    // first, and each lane copies its row out before the Pinv load reuses
    // the stage.
    const int r0 = chunk_r0(0);
    const int cvec = (min(64, n - r0) * W * (int)sizeof(T) + 15) / 16;
    unsigned char* st = reinterpret_cast<unsigned char*>(stage);
    constexpr int NVC = (64 * WC * (int)sizeof(T) + 1023) / 1024;
    auto dma_rows = [&](const T* __restrict__ gM) {
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(gM + (long long)r0 * W, (n - r0) * W * (int)sizeof(T));
#pragma unroll
      for (int u = 0; u < NVC; ++u) {
        if (lane + u * kWave < cvec)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(st + u * kWave * 16), 16,
              (lane + u * kWave) * 16, 0, 0, 0);
      }
    };
    if (a.resd_s_stage) {
      dma_rows(gS);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (valid[0]) {
        const T* __restrict__ m = stage + lane * W;
#pragma unroll
        for (int c = 0; c < WC; ++c) mS[0][c] = m[c];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    dma_rows(gP);
  }
  if constexpr (HYBS && kSViaLds) {
    // S chunks through the stage: coalesced direct loads, then each lane
    // copies its row into registers.
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      if (chunk_r0(k) < n) {  // wave-uniform
        dma_rows_to(gS, k, stage);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (valid[k]) {
          const T* __restrict__ m = stage_shift(gS, stage) + lane * W;
#pragma unroll
          for (int c = 0; c < WC; ++c) mS[k][c] = m[c];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    if (preg && a.preg_stage) {  // chunk 0 of Pinv the same way, into its registers
      dma_rows_to(gP, 0, stage);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (valid[0]) {
        const T* __restrict__ m = stage_shift(gP, stage) + lane * W;
#pragma unroll
        for (int c = 0; c < WC; ++c) mS[RPT - 1][c] = m[c];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
  // The first streamed Pinv chunk of the first pass into the stage (HYBS).
  if constexpr (HYBS) {
    int first = 0;
    while (first < RPT && !streams(first)) ++first;
    if (first < RPT) dma_chunk(first);
  }
  if (pin_last) dma_chunk_to(RPT - 1, pinned);
  dma_pinv_whole();
#pragma unroll
  for (int k = 0; k < RPT; ++k)
    if (valid[k]) p_pad[vix[k]] = xr[k];
  for (int e = tid; e < ssp; e += NT) {
    p_pad[e] = T(0);
    p_pad[(kp + 1) * ssp + e] = T(0);
    r_pad[e] = T(0);
    r_pad[(kp + 1) * ssp + e] = T(0);
  }
  block_sync();

  T sv[RPT];
  matvec(MatS{}, sv, mS, p_pad, Fwd{});  // S x0
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    rr[k] = valid[k] ? tmp[k] - sv[k] : T(0);
    if (valid[k]) r_pad[vix[k]] = rr[k];
  }
  // D blocks, or pinned chunks, landed
  if constexpr (HYBP) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (RESD) {
    // The wave's Pinv rows landed in its stage: each lane copies its own.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (valid[0]) {
      const T* __restrict__ m = stage + lane * W;
#pragma unroll
      for (int c = 0; c < WC; ++c) mP[0][c] = m[c];
    }
  }
  if constexpr (HYBS) {
    if (pin_last) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  block_sync();
  matvec(MatP{}, sv, mP, r_pad, Fwd{});  // z = Pinv r (pass 0)
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    pr[k] = sv[k];
    if (valid[k]) p_pad[vix[k]] = pr[k];  // p = z (x0 reads are done)
  }
  T rho = chunk_dot(rr, sv, slotA);  // also publishes p_pad
  const T rho0 = rho;
  const T rho_init = fabs(rho);
  const T thresh = mul_add_unfused(a.rel_tol, rho_init, a.abs_tol);
  T rho_last = rho;
  int iters = 0;
  int status = GLASS_PCG_MAX_ITERS;
  if (rho_init == T(0) || rho_init < thresh) {
    status = GLASS_PCG_CONVERGED;
  } else {
    for (int it = 0; it < a.max_iters; ++it) {
      matvec(MatS{}, sv, mS, p_pad, Fwd{});  // Sp
      const T pSp = chunk_dot(pr, sv, slotB);
      if (!(pSp > T(0)) || !is_finite_val(pSp)) {
        status = GLASS_PCG_BREAKDOWN;
        break;
      }
      const T alpha = rho / pSp;
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        xr[k] = fma(alpha, pr[k], xr[k]);
        rr[k] = fma(-alpha, sv[k], rr[k]);
        if (valid[k]) r_pad[vix[k]] = rr[k];
      }
      iters = it + 1;
      block_sync();
      // z = Pinv r (pass it + 1: odd passes walk the chunks backwards)
      if (HYBS && (it & 1) == 0) matvec(MatP{}, sv, mP, r_pad, Rev{});
      else matvec(MatP{}, sv, mP, r_pad, Fwd{});
      const T rz = chunk_dot(rr, sv, slotA);
      rho_last = rz;
      if (fabs(rz) < thresh) {
        status = GLASS_PCG_CONVERGED;
        break;
      }
      const T beta = rz / rho;
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        pr[k] = fma(beta, pr[k], sv[k]);
        if (valid[k]) p_pad[vix[k]] = pr[k];
      }
      rho = rz;
      block_sync();
    }
  }

#pragma unroll
  for (int k = 0; k < RPT; ++k)
    if (valid[k]) a.x[prob * n + row[k]] = xr[k];
  // Direct loads into LDS must land before the workgroup's LDS can pass to
  // another workgroup.  None is in flight here (the last chunk of a pass
  // starts no load); the wait makes sure.
  if constexpr (HYB) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (tid == 0) {
    if (a.iters) a.iters[prob] = iters;
    if (a.status) a.status[prob] = status;
    if (a.rho) {
      a.rho[2 * prob] = rho0;
      a.rho[2 * prob + 1] = rho_last;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Plan {
  int NW = 0;
  int RPT = 0;
  bool res = false;
  bool pd = false;  // Pinv's D blocks only (resident, or streamed with prefetch)
  bool packed = false;  // Pinv given as packed D blocks
  bool res_auto = false;  // resident rows per lane left to the occupancy choice
  bool resdma = false;    // resident, Pinv rows through the wave's LDS stage
  bool prefetch = false;
  bool hyb = false;  // S resident, Pinv streamed by direct loads into LDS
  int npin = 0;      // waves whose last Pinv chunk stays pinned in LDS
  bool regpin = false;  // waves without a last chunk hold chunk 0 of Pinv in registers
  int stage_elems = 0;
  size_t lds = 0;
};

template <typename T>
size_t lds_bytes(int ss, int kp, int NW, int stage_elems, bool padded = true) {
  const size_t nchunks = ((size_t)kp * ss + 63) / 64;
  const size_t head =
      ((size_t)(2 * (kp + 2) * vec_block<T>(ss, padded) + 2 * nchunks) * sizeof(T) + 15) &
      ~(size_t)15;
  return head + (size_t)NW * stage_elems * sizeof(T);
}

constexpr int kRptChoices[] = {1, 2, 3, 4, 8};

// Register-resident rows (S and Pinv, 3*ss each) fit in the 128-VGPR budget
// of a 1024-thread workgroup with room for the solver state.
template <typename T>
constexpr bool kResidentFits(int ss) {
  return 6 * ss * (int)sizeof(T) / 4 <= 96;
}
// The same budget when Pinv is block-diagonal (its rows hold ss values).
template <typename T>
constexpr bool kResidentFitsPD(int ss) {
  return 4 * ss * (int)sizeof(T) / 4 <= 96;
}
// Several resident rows per lane (workgroups of at most 8 waves, so up to
// 256 VGPRs per lane): rpt rows of S and Pinv within 176 registers.
template <typename T>
constexpr bool kResidentRowsFit(int ss, int rpt, bool pd) {
  return rpt * (pd ? 4 : 6) * ss * (int)sizeof(T) / 4 <= (rpt == 1 ? 96 : 176);
}

// HYBRID placement: built for the specialised sizes whose S and Pinv rows do
// not fit the one-row resident budget together; rpt rows of S alone within
// 192 registers (workgroups of at most 8 waves).
template <typename T>
constexpr bool kHybridSize(int ss) {
  return !kResidentFits<T>(ss);
}
template <typename T>
constexpr bool kHybridRowsFit(int ss, int rpt) {
  return kHybridSize<T>(ss) && rpt >= 1 && rpt <= 3 && rpt * 3 * ss * (int)sizeof(T) / 4 <= 192;
}

// Streamed with prefetch: specialised sizes whose 64-row chunk is at most 16
// 16-byte vectors per lane.
template <typename T>
constexpr bool kPrefetchFits(int ss) {
  return 3 * ss * (int)sizeof(T) <= 256;
}

// Elements of one wave's LDS stage for the prefetching placement: a whole
// number of 16-byte vectors per lane.
template <typename T>
int prefetch_stage_elems(int ss) {
  const int nv = (3 * ss * (int)sizeof(T) + 15) / 16;
  return nv * 64 * 16 / (int)sizeof(T);
}

// res_available: specialised size (resident rows possible); prefetch: the
// prefetching streamed placement is allowed (specialised, 16-byte aligned).
template <typename T>
bool make_plan(int ss, int kp, bool res_available, bool prefetch, bool pinv_diag,
               bool hybrid, bool pinv_packed, size_t lds_max, Plan* plan,
               bool prefetch_ok_for_dma = false) {
  const int n = kp * ss;
  const int W = 3 * ss;
  const int nchunks = (n + 63) / 64;
  // Register-resident rows when they fit comfortably in the VGPR budget:
  // one row per lane (up to 16 waves), or GLASS_AMD_PCG_RES_RPT rows per lane
  // (up to 8 waves; 2..4).
  const int forced_res_rpt = env_int("GLASS_AMD_PCG_RES_RPT", 0);
  const int res_rpt = forced_res_rpt > 0 ? forced_res_rpt : 1;
  const int res_nw = (nchunks + res_rpt - 1) / res_rpt;
  const bool res_fits = res_available && res_rpt >= 1 && res_rpt <= 4 &&
                        res_nw * 64 <= max_threads_for(res_rpt, kResident) &&
                        kResidentRowsFit<T>(ss, res_rpt, pinv_diag);
  if (res_fits) {
    Plan p;
    p.NW = res_nw;
    p.RPT = res_rpt;
    p.res = true;
    p.res_auto = forced_res_rpt == 0;
    p.pd = pinv_diag;
    p.stage_elems = 0;
    p.lds = lds_bytes<T>(ss, kp, p.NW, 0);
    if (p.lds <= lds_max) {
      // One row per lane, a general Pinv and 16-byte aligned rows: the Pinv
      // rows can come through a 64-row LDS stage per wave (the launch keeps
      // it only where it does not cost occupancy).
      if (res_rpt == 1 && !pinv_diag && prefetch_ok_for_dma && env_flag("GLASS_AMD_PCG_RES_DMA", 1)) {
        const size_t lds_d = lds_bytes<T>(ss, kp, p.NW, 64 * W);
        if (lds_d <= lds_max) {
          p.resdma = true;
          p.stage_elems = 64 * W;
          p.lds = lds_d;
        }
      }
      *plan = p;
      return true;
    }
  }
  // HYBRID (16-byte aligned, specialised size; a general Pinv streamed, or
  // its D blocks held whole in LDS, packed or under the block-diagonal
  // hint): the fewest rows per lane whose workgroup and LDS fit.
  if (hybrid) {
    const bool pin_ok = tuning_getenv("GLASS_AMD_PCG_NO_PIN") == nullptr;
    for (int rpt = 1; rpt <= 3; ++rpt) {
      if (rpt * 3 * ss * (int)sizeof(T) / 4 > 192) break;
      int NW = (nchunks + rpt - 1) / rpt;
      if (NW * 64 > max_threads_for(rpt, kHybrid)) continue;
      // Streaming a general Pinv with several chunks per wave: one wave
      // more leaves some waves without a last chunk, whose registers then
      // hold a Pinv chunk; take it when that pins more chunks in all (LDS
      // slots below plus those registers).
      auto pins = [&](int nw) {
        const size_t used = lds_bytes<T>(ss, kp, nw, prefetch_stage_elems<T>(ss), true);
        if (used > lds_max) return -1;
        const size_t slot = (size_t)prefetch_stage_elems<T>(ss) * sizeof(T);
        int have_last = 0, reg = 0;
        for (int w = 0; w < nw; ++w) {
          const bool last = (w + (rpt - 1) * nw) * 64 < n;
          have_last += last ? 1 : 0;
          reg += !last && w * 64 < n ? 1 : 0;
        }
        return std::min<int>(have_last, (int)((lds_max - used) / slot)) + reg;
      };
      if (!pinv_diag && pin_ok && rpt >= 2 && (NW + 1) * 64 <= max_threads_for(rpt, kHybrid) &&
          NW * 64 < n && pins(NW + 1) > pins(NW))
        NW = NW + 1;
      // D blocks in LDS: n*ss elements in whole 1 KB pieces.
      const size_t dbytes = ((size_t)n * ss * sizeof(T) + 1023) & ~(size_t)1023;
      const int stage = pinv_diag ? 0 : prefetch_stage_elems<T>(ss);
      const size_t lds = pinv_diag ? lds_bytes<T>(ss, kp, NW, 0) + dbytes
                                   : lds_bytes<T>(ss, kp, NW, stage, true);
      if (lds > lds_max) continue;
      Plan p;
      p.NW = NW;
      p.RPT = rpt;
      p.hyb = true;
      p.pd = pinv_diag;
      p.stage_elems = stage;
      p.lds = lds;
      // Streaming Pinv with several chunks per wave: the LDS left over pins
      // the last chunk of as many waves as fit (of those that have one).
      if (!pinv_diag && rpt >= 2 && pin_ok) {
        p.regpin = true;
        const size_t slot = (size_t)stage * sizeof(T);
        int have_last = 0;
        for (int w = 0; w < NW; ++w) have_last += (w + (rpt - 1) * NW) * 64 < n ? 1 : 0;
        const int npin = std::min<int>(have_last, (int)((lds_max - lds) / slot));
        p.npin = npin;
        p.lds = lds + (size_t)npin * slot;
      }
      *plan = p;
      return true;
    }
  }
  // Streamed: the fewest idle chunk slots, then the most waves.  The
  // prefetching placement is tried first; without it, plain staging.
  // GLASS_AMD_PCG_RPT forces the rows per lane of the streamed placements
  // (tests and tuning; an impossible value leaves no plan).
  const int forced_rpt = env_int("GLASS_AMD_PCG_RPT", 0);
  for (int pf = prefetch ? 1 : 0; pf >= 0; --pf) {
    const int mode = pf ? kStreamPrefetch : kStream;
    bool found = false;
    Plan best;
    int best_waste = 1 << 30;
    for (int rpt : kRptChoices) {
      if (forced_rpt > 0 && rpt != forced_rpt) continue;
      const int NW = (nchunks + rpt - 1) / rpt;
      if (NW * 64 > max_threads_for(rpt, mode)) continue;
      const int stage = pf ? prefetch_stage_elems<T>(ss) : 64 * W;
      const size_t lds = lds_bytes<T>(ss, kp, NW, stage, false);
      if (lds > lds_max) continue;
      const int waste = NW * rpt - nchunks;
      if (!found || waste < best_waste || (waste == best_waste && NW > best.NW)) {
        found = true;
        best_waste = waste;
        best.NW = NW;
        best.RPT = rpt;
        best.res = false;
        best.pd = pinv_diag && pf != 0;  // only the prefetching placement uses it
        best.prefetch = pf != 0;
        best.stage_elems = stage;
        best.lds = lds;
      }
    }
    if (found) {
      *plan = best;
      return true;
    }
  }
  return false;
}

template <typename T, int SS, int RPT, int MODE>
int launch_one(const PcgArgs<T>& a_in, int n_problems, const Plan& pl,
               hipStream_t stream) {
  PcgArgs<T> a = a_in;
  a.lds_bytes = (unsigned)pl.lds;
  auto kern = pcg_batched_kernel<T, SS, RPT, MODE>;
  if (int rc = allow_dynamic_lds((const void*)kern, pl.lds)) return rc;
  if (env_int("GLASS_AMD_VERBOSE", 0) > 0) {
    int per_cu = 0;
    (void)kernel_occupancy((const void*)kern, pl.NW * 64, pl.lds, &per_cu);
    std::fprintf(stderr,
                 "glass pcg plan: ss=%d kp=%d mode=%d waves=%d rows/lane=%d "
                 "lds=%zu stage=%d pinned=%d workgroups/CU=%d\n",
                 a.ss, a.kp, MODE, pl.NW, RPT, pl.lds, a.stage_elems, a.npin, per_cu);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)n_problems), dim3(pl.NW * 64), pl.lds,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "pcg launch");
  return GLASS_OK;
}

template <typename T, int SS, int MODE>
int launch_rpt(const PcgArgs<T>& a, int n_problems, const Plan& pl,
               hipStream_t st) {
  switch (pl.RPT) {
    case 1: return launch_one<T, SS, 1, MODE>(a, n_problems, pl, st);
    case 2: return launch_one<T, SS, 2, MODE>(a, n_problems, pl, st);
    case 3: return launch_one<T, SS, 3, MODE>(a, n_problems, pl, st);
    case 4: return launch_one<T, SS, 4, MODE>(a, n_problems, pl, st);
    default: return launch_one<T, SS, 8, MODE>(a, n_problems, pl, st);
  }
}

// Resident placement: one instantiation per rows-per-lane count that fits.
// Left to itself (no GLASS_AMD_PCG_RES_RPT), a batch with more problems than
// CUs takes two rows per lane instead of one when that kernel fits more
// workgroups per CU (more problems in flight); a smaller batch keeps one row
// per lane (the most waves per problem, the shortest solve).
template <typename T, int SS, bool PD, bool PACKED>
int launch_res(const PcgArgs<T>& a_in, int n_problems, const Plan& pl_in, hipStream_t st) {
  constexpr int M = PACKED ? kResidentPDP : (PD ? kResidentPD : kResident);
  Plan pl = pl_in;
  PcgArgs<T> a = a_in;
  if constexpr (!PD && !PACKED && kResidentRowsFit<T>(SS, 1, false)) {
    if (pl.resdma) {
      // The Pinv stage only where it keeps the occupancy of the plain kernel.
      int per_d = 0, per_p = 0;
      const size_t lds_p = lds_bytes<T>(a.ss, a.kp, pl.NW, 0);
      if (allow_dynamic_lds((const void*)pcg_batched_kernel<T, SS, 1, kResidentDma>, pl.lds) ==
              GLASS_OK &&
          kernel_occupancy((const void*)pcg_batched_kernel<T, SS, 1, kResidentDma>, pl.NW * 64,
                           pl.lds, &per_d) == GLASS_OK &&
          kernel_occupancy((const void*)pcg_batched_kernel<T, SS, 1, kResident>, pl.NW * 64,
                           lds_p, &per_p) == GLASS_OK &&
          per_d >= per_p && per_d > 0)
        return launch_one<T, SS, 1, kResidentDma>(a, n_problems, pl, st);
      pl.resdma = false;
      pl.stage_elems = 0;
      pl.lds = lds_p;
      a.stage_elems = 0;
    }
  }
  if constexpr (kResidentRowsFit<T>(SS, 1, PD) && kResidentRowsFit<T>(SS, 2, PD)) {
    DeviceInfo dev;
    const int nchunks = (a.kp * SS + 63) / 64;
    const int nw2 = (nchunks + 1) / 2;
    if (pl.res_auto && pl.RPT == 1 && nw2 * 64 <= max_threads_for(2, M) &&
        current_device_info(&dev) == GLASS_OK && n_problems > dev.cu_count) {
      int per1 = 0, per2 = 0;
      if (kernel_occupancy((const void*)pcg_batched_kernel<T, SS, 1, M>, pl.NW * 64, pl.lds,
                           &per1) == GLASS_OK &&
          kernel_occupancy((const void*)pcg_batched_kernel<T, SS, 2, M>, nw2 * 64, pl.lds,
                           &per2) == GLASS_OK &&
          per2 > per1) {
        pl.RPT = 2;
        pl.NW = nw2;
      }
    }
  }
  switch (pl.RPT) {
    case 1:
      if constexpr (kResidentRowsFit<T>(SS, 1, PD)) return launch_one<T, SS, 1, M>(a, n_problems, pl, st);
      break;
    case 2:
      if constexpr (kResidentRowsFit<T>(SS, 2, PD)) return launch_one<T, SS, 2, M>(a, n_problems, pl, st);
      break;
    case 3:
      if constexpr (kResidentRowsFit<T>(SS, 3, PD)) return launch_one<T, SS, 3, M>(a, n_problems, pl, st);
      break;
    case 4:
      if constexpr (kResidentRowsFit<T>(SS, 4, PD)) return launch_one<T, SS, 4, M>(a, n_problems, pl, st);
      break;
    default:
      break;
  }
  return fail(GLASS_EUNSUPPORTED, "pcg: internal plan error (resident rows per lane)");
}

template <typename T, int SS, int M>
int launch_hyb(const PcgArgs<T>& a, int n_problems, const Plan& pl, hipStream_t st) {
  switch (pl.RPT) {
    case 1:
      if constexpr (kHybridRowsFit<T>(SS, 1)) return launch_one<T, SS, 1, M>(a, n_problems, pl, st);
      break;
    case 2:
      if constexpr (kHybridRowsFit<T>(SS, 2)) return launch_one<T, SS, 2, M>(a, n_problems, pl, st);
      break;
    case 3:
      if constexpr (kHybridRowsFit<T>(SS, 3)) return launch_one<T, SS, 3, M>(a, n_problems, pl, st);
      break;
    default:
      break;
  }
  return fail(GLASS_EUNSUPPORTED, "pcg: internal plan error (hybrid rows per lane)");
}

template <typename T, int SS>
int launch_ss(const PcgArgs<T>& a, int n_problems, const Plan& pl,
              hipStream_t st) {
  if constexpr (SS > 0) {
    if (pl.hyb)
      return !pl.pd ? launch_hyb<T, SS, kHybrid>(a, n_problems, pl, st)
                    : (pl.packed ? launch_hyb<T, SS, kHybridPDP>(a, n_problems, pl, st)
                                 : launch_hyb<T, SS, kHybridPD>(a, n_problems, pl, st));
    if (pl.res) {
      if (!pl.pd) return launch_res<T, SS, false, false>(a, n_problems, pl, st);
      return pl.packed ? launch_res<T, SS, true, true>(a, n_problems, pl, st)
                       : launch_res<T, SS, true, false>(a, n_problems, pl, st);
    }
  }
  if constexpr (SS > 0 && kPrefetchFits<T>(SS)) {
    if (pl.prefetch)
      return pl.pd ? (pl.packed ? launch_rpt<T, SS, kStreamPrefetchPDP>(a, n_problems, pl, st)
                                : launch_rpt<T, SS, kStreamPrefetchPD>(a, n_problems, pl, st))
                   : launch_rpt<T, SS, kStreamPrefetch>(a, n_problems, pl, st);
  }
  return launch_rpt<T, SS, kStream>(a, n_problems, pl, st);
}

// 16-byte vector paths: S and Pinv 16-byte aligned and every problem's
// matrices starting on a 16-byte boundary.
template <typename T>
bool vector_ok(const void* S, const void* P, int ss, int kp, bool pinv_packed) {
  const long long n = (long long)kp * ss, es = (long long)sizeof(T);
  return aligned(S, 16) && aligned(P, 16) && (n * 3 * ss * es) % 16 == 0 &&
         (!pinv_packed || (n * ss * es) % 16 == 0);
}

// The plan for a shape.  GLASS_AMD_PCG_STREAMED=1 replaces a resident plan
// by a streamed one (tests and measurement); it keeps the D-block hint only
// for packed D blocks, which the general streamed modes cannot read.  A
// packed Pinv is only ever given to the D-block modes or kStream.
template <typename T>
bool choose_plan(int ss, int kp, bool vec, bool pinv_diag, bool pinv_packed, size_t lds_max,
                 Plan* pl) {
  const bool specialised = ss == 6 || ss == 12 || ss == 14 || ss == 21;
  const bool prefetch = specialised && vec && kPrefetchFits<T>(ss) &&
                        tuning_getenv("GLASS_AMD_PCG_NO_PREFETCH") == nullptr;
  // S resident with Pinv streamed also takes matrices aligned to the element
  // size only (its chunk loads shift, see the kernel), where a 64-row chunk
  // leaves spare bytes in the stage (3ss elements not a multiple of 16 bytes);
  // the D-block variants need 16-byte alignment.
  const bool shiftable = (3 * ss * (int)sizeof(T)) % 16 != 0 && !pinv_diag && !pinv_packed;
  const bool hybrid = specialised && (vec || shiftable) && kHybridSize<T>(ss) &&
                      tuning_getenv("GLASS_AMD_PCG_NO_HYBRID") == nullptr;
  pinv_diag = pinv_diag || pinv_packed;
  if (!make_plan<T>(ss, kp, specialised, prefetch, pinv_diag, hybrid, pinv_packed, lds_max, pl,
                    specialised && vec))
    return false;
  if (const char* f = tuning_getenv("GLASS_AMD_PCG_STREAMED"); f && f[0] == '1' && (pl->res || pl->hyb)) {
    Plan alt;
    if (make_plan<T>(ss, kp, false, prefetch, pinv_packed, false, pinv_packed, lds_max, &alt))
      *pl = alt;
  }
  if (pinv_packed && !pl->pd && (pl->res || pl->prefetch)) return false;  // not reached
  pl->packed = pinv_packed;
  return true;
}

// Several problems per wave (pcg_multi.hip) for the small shapes it covers
// with Pinv in [L|D|R] form.  Chosen by itself where it was measured faster
// than the workgroup placement: chains of at most 16 rows (one row per lane,
// four problems per wave; 1.2-2.4x at kp = 1-2).  With more rows per lane
// each lane's serial chain outweighs the barriers it saves (measured slower
// at kp = 4-32).  GLASS_AMD_PCG_MULTI=1 selects it wherever it fits, 0 never.
bool use_multi(glass_dtype dt, int ss, int kp, bool pinv_packed) {
  if (pinv_packed || !pcg_multi_fits(dt, ss, kp)) return false;
  return env_flag("GLASS_AMD_PCG_MULTI", (long long)kp * ss <= 16 ? 1 : 0) == 1;
}

template <typename T>
int launch_typed(T* x, const T* S, const T* P, const T* b, int ss, int kp,
                 int n_problems, int max_iters, double rel_tol, double abs_tol,
                 int* iters, int* status, T* rho, bool pinv_diag, bool pinv_packed,
                 hipStream_t st) {
  constexpr glass_dtype dt = sizeof(T) == 4 ? GLASS_F32 : GLASS_F64;
  if (use_multi(dt, ss, kp, pinv_packed))
    return launch_pcg_multi(dt, x, S, P, b, ss, kp, n_problems, max_iters, rel_tol, abs_tol,
                            iters, status, rho, st);
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  const bool vec = vector_ok<T>(S, P, ss, kp, pinv_packed);
  Plan pl;
  if (!choose_plan<T>(ss, kp, vec, pinv_diag, pinv_packed, dev.max_lds_per_block, &pl))
    return fail(GLASS_EUNSUPPORTED,
                "pcg: problem too large for one workgroup (rows or LDS)");
  PcgArgs<T> a;
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
  a.vec = vec;
  a.stage_elems = pl.stage_elems;
  a.npin = pl.npin;
  a.regpin = pl.regpin ? 1 : 0;
  a.ppacked = pinv_packed ? 1 : 0;
  // Rows of 128 bytes or more: one load instruction of a lane's own S row
  // touches as many cache lines as the wave has lanes, so the coalesced
  // staging wins (ss=14 fp32: 168-byte rows); shorter rows load directly.
  a.resd_s_stage =
      env_flag("GLASS_AMD_PCG_RESD_S_STAGE", 3 * ss * (int)sizeof(T) >= 128 ? 1 : 0);
  a.preg_stage = env_flag("GLASS_AMD_PCG_PREG_STAGE", 1);
  switch (ss) {
    case 6: return launch_ss<T, 6>(a, n_problems, pl, st);
    case 12: return launch_ss<T, 12>(a, n_problems, pl, st);
    case 14: return launch_ss<T, 14>(a, n_problems, pl, st);
    case 21: return launch_ss<T, 21>(a, n_problems, pl, st);
    default: return launch_ss<T, 0>(a, n_problems, pl, st);
  }
}

template <typename T>
int placement_typed(int ss, int kp, bool aligned16, bool pinv_diag, bool pinv_packed) {
  constexpr glass_dtype dt = sizeof(T) == 4 ? GLASS_F32 : GLASS_F64;
  if (use_multi(dt, ss, kp, pinv_packed)) return GLASS_PLACEMENT_SEVERAL_PER_WAVE;
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  const long long n = (long long)kp * ss, es = (long long)sizeof(T);
  const bool vec = aligned16 && (n * 3 * ss * es) % 16 == 0 &&
                   (!pinv_packed || (n * ss * es) % 16 == 0);
  Plan pl;
  if (!choose_plan<T>(ss, kp, vec, pinv_diag, pinv_packed, dev.max_lds_per_block, &pl))
    return fail(GLASS_EUNSUPPORTED, "pcg: problem too large for one workgroup (rows or LDS)");
  // S in registers with the D blocks in LDS reads both once.
  if (pl.hyb) return pl.pd ? GLASS_PLACEMENT_RESIDENT : GLASS_PLACEMENT_S_RESIDENT;
  return pl.res ? GLASS_PLACEMENT_RESIDENT
                : (pl.prefetch ? GLASS_PLACEMENT_STREAMED_PREFETCH : GLASS_PLACEMENT_STREAMED);
}

template <typename T>
int pinned_rows_typed(int ss, int kp, bool aligned16, bool pinv_diag, bool pinv_packed) {
  constexpr glass_dtype dt = sizeof(T) == 4 ? GLASS_F32 : GLASS_F64;
  if (use_multi(dt, ss, kp, pinv_packed)) return 0;
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  const long long n = (long long)kp * ss, es = (long long)sizeof(T);
  const bool vec = aligned16 && (n * 3 * ss * es) % 16 == 0 &&
                   (!pinv_packed || (n * ss * es) % 16 == 0);
  Plan pl;
  if (!choose_plan<T>(ss, kp, vec, pinv_diag, pinv_packed, dev.max_lds_per_block, &pl))
    return fail(GLASS_EUNSUPPORTED, "pcg: problem too large for one workgroup (rows or LDS)");
  int rows = 0;
  for (int w = 0; w < pl.npin; ++w) {
    const long long r0 = (long long)(w + (pl.RPT - 1) * pl.NW) * 64;
    rows += (int)std::min<long long>(64, n - r0);
  }
  if (pl.regpin && pl.RPT >= 2) {  // chunk 0 of waves without a last chunk
    for (int w = 0; w < pl.NW; ++w)
      if ((long long)(w + (pl.RPT - 1) * pl.NW) * 64 >= n && (long long)w * 64 < n)
        rows += (int)std::min<long long>(64, n - (long long)w * 64);
  }
  return rows;
}

// Pinv rows (per problem) that matvec pass `pass` reads from memory: the
// plan's chunk walk as the kernel does it (pass 0 forward and the pinned
// rows once; then alternate directions, each pass starting with the chunk
// the previous one left in the wave's stage).
template <typename T>
int pass_rows_typed(int ss, int kp, bool aligned16, bool pinv_diag, bool pinv_packed, int pass) {
  constexpr glass_dtype dt = sizeof(T) == 4 ? GLASS_F32 : GLASS_F64;
  const long long n = (long long)kp * ss, es = (long long)sizeof(T);
  if (use_multi(dt, ss, kp, pinv_packed)) return pass == 0 ? (int)n : 0;
  DeviceInfo dev;
  if (int rc = current_device_info(&dev)) return rc;
  const bool vec = aligned16 && (n * 3 * ss * es) % 16 == 0 &&
                   (!pinv_packed || (n * ss * es) % 16 == 0);
  Plan pl;
  if (!choose_plan<T>(ss, kp, vec, pinv_diag, pinv_packed, dev.max_lds_per_block, &pl))
    return fail(GLASS_EUNSUPPORTED, "pcg: problem too large for one workgroup (rows or LDS)");
  if (!pl.hyb) return pl.res ? (pass == 0 ? (int)n : 0) : (int)n;
  if (pl.pd) return pass == 0 ? (int)n : 0;  // D blocks in LDS, read once
  long long rows = 0;
  for (int w = 0; w < pl.NW; ++w) {
    auto chunk_rows = [&](int k) -> long long {
      const long long r0 = (long long)(w + k * pl.NW) * 64;
      return r0 < n ? std::min<long long>(64, n - r0) : 0;
    };
    const bool pin_last = w < pl.npin;
    const bool preg = pl.regpin && pl.RPT >= 2 && chunk_rows(pl.RPT - 1) == 0 && chunk_rows(0) > 0;
    auto streams = [&](int k) {
      const bool off = (pin_last && k == pl.RPT - 1) || (preg && k == 0);
      return !off && chunk_rows(k) > 0;
    };
    int first = -1, last = -1;
    long long streamed = 0;
    for (int k = 0; k < pl.RPT; ++k)
      if (streams(k)) {
        if (first < 0) first = k;
        last = k;
        streamed += chunk_rows(k);
      }
    if (pass == 0) {
      rows += streamed;
      if (pin_last) rows += chunk_rows(pl.RPT - 1);
      if (preg) rows += chunk_rows(0);
    } else if (first >= 0) {
      rows += streamed - chunk_rows((pass & 1) ? last : first);
    }
  }
  return (int)rows;
}

}  // namespace

int pcg_batched_pinv_pass_rows(glass_dtype dt, int ss, int kp, bool aligned16, bool pinv_diag,
                               bool pinv_packed, int pass) {
  return dt == GLASS_F32
             ? pass_rows_typed<float>(ss, kp, aligned16, pinv_diag, pinv_packed, pass)
             : pass_rows_typed<double>(ss, kp, aligned16, pinv_diag, pinv_packed, pass);
}

int pcg_batched_pinned_rows(glass_dtype dt, int ss, int kp, bool aligned16, bool pinv_diag,
                            bool pinv_packed) {
  return dt == GLASS_F32 ? pinned_rows_typed<float>(ss, kp, aligned16, pinv_diag, pinv_packed)
                         : pinned_rows_typed<double>(ss, kp, aligned16, pinv_diag, pinv_packed);
}

int pcg_batched_placement(glass_dtype dt, int ss, int kp, bool aligned16, bool pinv_diag,
                          bool pinv_packed) {
  return dt == GLASS_F32 ? placement_typed<float>(ss, kp, aligned16, pinv_diag, pinv_packed)
                         : placement_typed<double>(ss, kp, aligned16, pinv_diag, pinv_packed);
}

int launch_pcg_batched(glass_dtype dt, void* x, const void* S,
                       const void* Pinv, const void* b, int ss, int kp,
                       int n_problems, int max_iters, double rel_tol,
                       double abs_tol, int* iters, int* status, void* rho,
                       bool pinv_diag, bool pinv_packed, hipStream_t stream) {
  if (dt == GLASS_F32)
    return launch_typed<float>((float*)x, (const float*)S, (const float*)Pinv,
                               (const float*)b, ss, kp, n_problems, max_iters,
                               rel_tol, abs_tol, iters, status, (float*)rho,
                               pinv_diag, pinv_packed, stream);
  return launch_typed<double>((double*)x, (const double*)S,
                              (const double*)Pinv, (const double*)b, ss, kp,
                              n_problems, max_iters, rel_tol, abs_tol, iters,
                              status, (double*)rho, pinv_diag, pinv_packed, stream);
}

}  // namespace glass
