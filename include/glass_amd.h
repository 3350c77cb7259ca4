/*
 * glass_amd.h -- C ABI of the MI355X (gfx950) batched block-tridiagonal
 * matvec and preconditioned conjugate-gradient library.
 *
 * Operations (GLASS user guide, page "Block-tridiagonal Solves"):
 *   - section "The [L|D|R] block-tridiagonal layout": a block-tridiagonal
 *     matrix with knot_points block-rows of size state_size is stored as
 *     knot_points contiguous row-major strips, each state_size x 3*state_size,
 *     holding [L_br | D_br | R_br]; L of the first and R of the last block-row
 *     are stored but multiply zero pads.
 *   - section "The padded vector layout": vectors of (knot_points+2)*state_size
 *     with one zero pad block at each end; block-row br reads the window
 *     v[br*ss, br*ss + 3*ss) and writes y[(br+1)*ss + row].
 *   - section "Matvec -- glass::bdmv": y = A_bd * v.
 *   - section "Solve -- glass::pcg": preconditioned CG on S x = b with a
 *     block-tridiagonal preconditioner Pinv (also in [L|D|R] form); stop when
 *     |rho| < abs_tol + rel_tol * |rho_init| with rho = r^T z the
 *     preconditioned residual; x carries the initial guess in and the
 *     solution out; the iteration count is returned.
 *   - the same page names a cooperative grid-wide PCG (one solve spanning the
 *     whole grid) as future work; glass_pcg_grid is that solve.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller (e.g. torch
 *     tensors).  Nothing is allocated or freed by the library.
 *   - Work is enqueued asynchronously on hip_stream (a hipStream_t; NULL is
 *     the null stream).  No entry point synchronises the host.
 *   - dtype selects float (GLASS_F32) or double (GLASS_F64) for every
 *     floating-point array of the call.
 *   - Layouts are problem-major and contiguous:
 *       S, Pinv   [n_problems][knot_points][state_size][3*state_size]
 *       bdmv v, y [n_problems][(knot_points+2)*state_size]   (padded)
 *       PCG x, b  [n_problems][knot_points*state_size]        (unpadded)
 *       iters_out, status_out   int32 [n_problems]
 *       rho_out   dtype [n_problems][2] = (signed initial r^T z, last r^T z)
 *   - Base pointers must be aligned to the element size; 16-byte alignment
 *     enables the vectorised loads (otherwise a scalar path is used).
 *   - Return value: GLASS_OK, or a negative GLASS_E* code; on error nothing
 *     has been enqueued (except GLASS_EHIP, which reports a failed launch).
 *     glass_last_error() then describes the failure (per host thread).
 *   - Calls on one stream run in order; calls on different streams that write
 *     the same memory race, as with any HIP kernel.
 *   - The library reads no environment variable, except in a process that
 *     sets GLASS_AMD_TUNING=1 before its first call: there its test and
 *     tuning switches (GLASS_AMD_* names) can force placements and launch
 *     shapes.
 */
#ifndef GLASS_AMD_H
#define GLASS_AMD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the floating-point arrays.  In C++ the enum has a fixed
 * int underlying type, so any int a C caller passes is a value of the type
 * (and the library rejects the others with GLASS_EINVAL) rather than
 * undefined behaviour; the ABI is an int either way. */
#ifdef __cplusplus
typedef enum : int { GLASS_F32 = 0, GLASS_F64 = 1 } glass_dtype;
#else
typedef enum { GLASS_F32 = 0, GLASS_F64 = 1 } glass_dtype;
#endif

enum {
  GLASS_OK = 0,
  GLASS_EINVAL = -1,       /* null pointer, size <= 0, bad dtype, misaligned,
                              max_iters < 0, tolerance negative or NaN */
  GLASS_EUNSUPPORTED = -2, /* valid, but beyond this build's size limits */
  GLASS_EHIP = -3,         /* a HIP runtime call or launch failed */
  GLASS_ECOOP = -4         /* the grid solve cannot be made co-resident */
};

/* Per-problem PCG outcome written to status_out. */
enum {
  GLASS_PCG_CONVERGED = 0, /* |rho| < abs_tol + rel_tol*|rho_init| was met
                              (also when rho_init == 0: nothing to do)   */
  GLASS_PCG_MAX_ITERS = 1, /* max_iters iterations ran without meeting it   */
  GLASS_PCG_BREAKDOWN = 2, /* p^T S p <= 0 or not finite (S not SPD, NaN);
                              x keeps the last completed update           */
  GLASS_PCG_GRID_TIMEOUT = 3 /* glass_pcg_grid only: a grid barrier wait
                              gave up (workgroups not co-resident after
                              all); the kernel drained, x is unreliable   */
};

/* Per-problem outcome of glass_bdsv_batched written to status_out. */
enum {
  GLASS_BDSV_OK = 0,      /* solved                                           */
  GLASS_BDSV_NOT_SPD = 1  /* a pivot block (Schur complement) is not
                             numerically positive definite; x is unchanged   */
};

/* Largest state_size accepted by any entry point. */
#define GLASS_MAX_STATE_SIZE 64
/* Largest state_size accepted by glass_bdsv_batched. */
#define GLASS_BDSV_MAX_STATE_SIZE 24

/*
 * y = A_bd * v for n_problems independent matrices (page "Block-tridiagonal
 * Solves", sections "The padded vector layout" and "Matvec -- glass::bdmv"):
 *   y[q][(br+1)*ss + i] = sum_{c < 3ss} S[q][br][i][c] * v[q][br*ss + c]
 * for br < knot_points, i < state_size.  The caller zeroes the pad blocks of
 * v; the pad blocks of y are not written.  y must not overlap S or v.
 * Each output row is summed by one thread in a fixed order, so the result does
 * not depend on the launch shape.
 * Limits: 1 <= state_size <= GLASS_MAX_STATE_SIZE, knot_points >= 1,
 * n_problems >= 0 (0 enqueues nothing).
 */
int glass_bdmv_batched(void* y, const void* S, const void* v, int state_size,
                       int knot_points, int n_problems, glass_dtype dtype,
                       void* hip_stream);

/*
 * Preconditioned conjugate gradient on S x = b, one independent problem per
 * workgroup (page "Block-tridiagonal Solves", section "Solve -- glass::pcg").
 * On entry x holds the initial guess; on exit the solution.  Steps:
 *   r = b - S x; z = Pinv r; p = z; rho = r^T z; rho_init = |rho|;
 *   thresh = abs_tol + rel_tol * rho_init (both rounded to dtype);
 *   converged at once if rho_init == 0 or rho_init < thresh; otherwise per
 *   iteration: Sp = S p; alpha = rho / (p^T Sp); x += alpha p;
 *   r -= alpha Sp; z = Pinv r; rho' = r^T z; stop if |rho'| < thresh;
 *   p = z + (rho'/rho) p; rho = rho'.
 * iters_out[q] = number of completed x updates (<= max_iters).  S and Pinv
 * must be symmetric positive definite for the result to be meaningful; a
 * non-positive p^T S p stops that problem with GLASS_PCG_BREAKDOWN.
 * Limits: state_size <= GLASS_MAX_STATE_SIZE; knot_points*state_size <= 8192
 * rows.  When S and Pinv do not stay in registers they are staged through a
 * 64-row LDS chunk per wave, which must fit in LDS next to two padded
 * vectors: in float32 that allows up to about 4000 rows at state_size 12-21
 * and 8190 at state_size 6.  Larger shapes return GLASS_EUNSUPPORTED before
 * anything is launched (glass_pcg_batched_placement reports it too).
 */
int glass_pcg_batched(void* x, const void* S, const void* Pinv, const void* b,
                      int state_size, int knot_points, int n_problems,
                      int max_iters, double rel_tol, double abs_tol,
                      int* iters_out, glass_dtype dtype, void* hip_stream);

/* As glass_pcg_batched, plus optional per-problem outputs (either may be
 * NULL): status_out (GLASS_PCG_*) and rho_out (see conventions), and flags:
 *   GLASS_PCG_PINV_BLOCK_DIAGONAL  the caller asserts that the L and R blocks
 *     of every block-row of Pinv are zero (a block-Jacobi preconditioner,
 *     one of the choices the same page names).  Pinv keeps its [L|D|R]
 *     layout.  Where each lane keeps its rows in registers only the D blocks
 *     are requested and held (fewer registers, a third of Pinv's
 *     multiply-adds); where rows are streamed, 16-byte pieces that touch no
 *     D block are not requested.  Memory traffic shrinks only where whole
 *     cache lines lie outside the D blocks.  When the assertion holds the results are the
 *     same as without the flag (the skipped terms are exact zeros, added in
 *     the same order); when it does not, the L and R blocks of Pinv may or
 *     may not be used.
 *   GLASS_PCG_PINV_DIAGONAL_BLOCKS  Pinv holds only the D blocks, packed:
 *     [n_problems][kp][ss][ss] row-major (row i of block-row br starts at
 *     element (br*ss + i)*ss of its problem), kp*ss*ss elements per problem
 *     instead of kp*ss*3ss.  The same block-Jacobi preconditioner as
 *     GLASS_PCG_PINV_BLOCK_DIAGONAL (which it implies), with every placement
 *     reading a third of Pinv's bytes.  The results are the same as for the
 *     [L|D|R] layout with zero L and R blocks (the same terms in the same
 *     order).  Alignment as for S: the element size, 16 bytes for the
 *     vector paths.
 * Other flag bits return GLASS_EINVAL. */
enum { GLASS_PCG_PINV_BLOCK_DIAGONAL = 1u, GLASS_PCG_PINV_DIAGONAL_BLOCKS = 2u };
int glass_pcg_batched_ex(void* x, const void* S, const void* Pinv,
                         const void* b, int state_size, int knot_points,
                         int n_problems, int max_iters, double rel_tol,
                         double abs_tol, int* iters_out, int* status_out,
                         void* rho_out, glass_dtype dtype, unsigned flags,
                         void* hip_stream);

/* Where glass_pcg_batched_ex keeps S and Pinv for a problem shape and flags
 * on the current device: GLASS_PLACEMENT_RESIDENT (both read from HBM once
 * per solve: each lane's rows in registers, or for packed D blocks that do
 * not fit there, S's rows in registers and the D blocks in LDS),
 * GLASS_PLACEMENT_STREAMED[_PREFETCH] (re-read from memory for every
 * matvec) or GLASS_PLACEMENT_S_RESIDENT (S's rows in registers, read once;
 * Pinv re-read for every matvec through the LDS; matrices aligned to the
 * element size are enough where a row of 3*state_size elements is not a
 * multiple of 16 bytes, else they must be 16-byte aligned).  Every placement gives the same bits.  aligned16: whether S and Pinv will be 16-byte aligned.  flags:
 * as glass_pcg_batched_ex (0 for glass_pcg_batched).  Returns a negative
 * GLASS_E* code for shapes the solve rejects.  Enqueues nothing. */
enum {
  GLASS_PLACEMENT_RESIDENT = 0,
  GLASS_PLACEMENT_STREAMED_PREFETCH = 1,
  GLASS_PLACEMENT_STREAMED = 2,
  GLASS_PLACEMENT_S_RESIDENT = 3,
  GLASS_PLACEMENT_SEVERAL_PER_WAVE = 4  /* small problems (state_size 6, up to
                                           192 rows; Pinv in [L|D|R] form):
                                           16 or 32 lanes per problem, 4 or 2
                                           problems per wave, S and Pinv rows
                                           in registers (read once), no
                                           workgroup barriers */
};
int glass_pcg_batched_placement(int state_size, int knot_points,
                                glass_dtype dtype, int aligned16, unsigned flags);

/* In GLASS_PLACEMENT_S_RESIDENT, the number of Pinv strip rows (per problem)
 * that stay on chip for the whole solve: the LDS left over after the
 * per-wave stages holds the last chunk of 64 rows of some waves, and waves
 * with a register row to spare hold their first chunk there; these are read
 * from memory once.  0 for the other placements.  Arguments, errors and side
 * effects as glass_pcg_batched_placement (it enqueues nothing). */
int glass_pcg_batched_pinned_rows(int state_size, int knot_points,
                                  glass_dtype dtype, int aligned16, unsigned flags);

/* The number of Pinv strip rows (per problem) that matvec pass `pass` reads
 * from memory on the current device: pass 0 is z = Pinv r0 and also counts
 * the rows kept on chip for the whole solve; pass p >= 1 is iteration p's
 * z = Pinv r.  In GLASS_PLACEMENT_S_RESIDENT the other rows stream through
 * one LDS stage per wave, in 64-row chunks; passes walk each wave's chunks in
 * alternating directions, so a pass after the first starts with the chunk
 * the previous pass left in the stage and does not read it again (the count
 * then alternates between odd and even passes when a chunk is short).
 * Resident placements: knot_points*state_size rows at pass 0, 0 after;
 * streamed placements: knot_points*state_size at every pass.  pass < 0 is
 * GLASS_EINVAL; otherwise arguments, errors and side effects as
 * glass_pcg_batched_placement (it enqueues nothing). */
int glass_pcg_batched_pinv_pass_rows(int state_size, int knot_points,
                                     glass_dtype dtype, int aligned16, unsigned flags,
                                     int pass);

/*
 * One PCG solve (same steps and outputs as glass_pcg_batched with
 * n_problems = 1) spread over a cooperative grid of workgroups that stay
 * co-resident on the device; each workgroup owns a contiguous range of
 * block-rows, and the dot products are reduced across the grid in a fixed
 * order, so every workgroup takes identical decisions.
 * workspace: caller-owned device memory of at least
 * glass_pcg_grid_workspace_bytes(...) bytes, 256-byte aligned; its contents on
 * entry do not matter and it must not be used by another call on another
 * stream at the same time.
 * Limits: knot_points >= 4; state_size <= GLASS_MAX_STATE_SIZE.
 * Returns GLASS_ECOOP if the device cannot hold a large enough grid.
 *
 * glass_pcg_grid launches through the runtime's cooperative launch, which
 * guarantees co-residency on a shared device.  glass_pcg_grid_ex takes flags:
 *   0                     the same cooperative launch;
 *   GLASS_GRID_EXCLUSIVE  an ordinary dispatch on hip_stream's own queue,
 *     about 20 us cheaper per solve on MI355X.  The same co-residency check
 *     runs on the host (the whole grid fits on the device at once), but the
 *     caller vouches that no kernel from another stream or process occupies
 *     compute units while the solve runs.  If that is broken and workgroups
 *     cannot all start, the bounded barrier waits expire and the solve
 *     reports GLASS_PCG_GRID_TIMEOUT (after up to a few seconds) instead of
 *     hanging; x is then unspecified.
 *   GLASS_GRID_SINGLE_REDUCTION  the single-reduction form of PCG
 *     (Chronopoulos and Gear, preconditioned): u = Pinv r and w = S u are
 *     carried by recurrences, so r^T u and w^T u are reduced together and
 *     each iteration needs one grid-wide reduction instead of two.  In exact
 *     arithmetic it has the same iterates, stopping rule, iteration count,
 *     breakdown test (its step denominator equals p^T S p) and outputs as the
 *     steps above; in floating point it rounds differently.  It holds S and
 *     Pinv rows for one more block-row on each side of a workgroup's range.
 *   GLASS_GRID_KEEP_WORKSPACE  the caller keeps this workspace for grid
 *     solves: between this call and the previous grid solve given the same
 *     workspace address on this device, nothing else wrote it.  The library
 *     then skips the per-solve clearing of its exchange words (one small
 *     kernel launch, about 4 us per solve on MI355X): the host remembers, per
 *     address, which tags earlier solves may have left and starts this
 *     solve's tags above them.  The first kept solve at an address, and one
 *     about every 2^32 grid barriers, still clears the whole workspace.
 *     Without the flag the workspace contents on entry do not matter.
 * Other flag bits return GLASS_EINVAL.
 */
enum {
  GLASS_GRID_EXCLUSIVE = 1u,
  GLASS_GRID_SINGLE_REDUCTION = 2u,
  GLASS_GRID_KEEP_WORKSPACE = 4u
};
size_t glass_pcg_grid_workspace_bytes(int state_size, int knot_points,
                                      glass_dtype dtype);
int glass_pcg_grid(void* x, const void* S, const void* Pinv, const void* b,
                   int state_size, int knot_points, int max_iters,
                   double rel_tol, double abs_tol, int* iters_out,
                   void* workspace, size_t workspace_bytes, glass_dtype dtype,
                   void* hip_stream);
int glass_pcg_grid_ex(void* x, const void* S, const void* Pinv, const void* b,
                      int state_size, int knot_points, int max_iters,
                      double rel_tol, double abs_tol, int* iters_out,
                      int* status_out, void* rho_out, void* workspace,
                      size_t workspace_bytes, glass_dtype dtype,
                      unsigned flags, void* hip_stream);

/*
 * glass_pcg_grid_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus workspace and
 * workspace_bytes), flags, steps, outputs and results (bit for bit) as
 * glass_pcg_grid_ex; the array is always kept for grid solves (as with
 * GLASS_GRID_KEEP_WORKSPACE), so after its first call on a device no
 * clearing kernel is launched.  The exchange area lives in a static device array of
 * GLASS_PCG_GRID_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * device it runs on until the process ends; the call itself allocates and
 * frees nothing.  It needs 256 + 8*2*G*64 + 2*G*4*state_size*w*8 bytes
 * (G = workgroups of the grid, usually one per compute unit; w = 1 for
 * GLASS_F32, 2 for GLASS_F64), about 0.66 MB for a 256-workgroup fp64 grid
 * at state_size 12; a shape that needs more returns GLASS_EUNSUPPORTED with
 * nothing launched.  Every call on one device shares that device's array:
 * calls ordered on one stream are safe, calls that overlap in time (other
 * streams, other host threads) race and give unspecified results.
 */
#define GLASS_PCG_GRID_NOALLOC_SCRATCH_BYTES 4194304
int glass_pcg_grid_noalloc(void* x, const void* S, const void* Pinv,
                           const void* b, int state_size, int knot_points,
                           int max_iters, double rel_tol, double abs_tol,
                           int* iters_out, int* status_out, void* rho_out,
                           glass_dtype dtype, unsigned flags, void* hip_stream);

/*
 * Direct solve S x = b for n_problems independent block-tridiagonal
 * symmetric positive definite systems (glass::bdsv, named in the opening
 * paragraph of page "Block-tridiagonal Solves"; layout as above).  Steps:
 * block elimination without pivoting across block-rows,
 *   [M_br | y_br] = [D_br | b_br] - L_br [G_{br-1} | u_{br-1}]   (br > 0),
 *   [G_br | u_br] = M_br^{-1} [R_br | y_br]   (no R for the last block-row),
 *   x_{kp-1} = u_{kp-1},  x_br = u_br - G_br x_{br+1},
 * each pivot block M_br (a Schur complement, SPD when S is SPD) eliminated
 * with positive diagonal pivots.  S must be symmetric (R_br = L_{br+1}^T);
 * otherwise the result is unspecified.  L of the first and R of the last
 * block-row are ignored.
 * x, b: [n_problems][knot_points*state_size] (unpadded); x is written only
 * for problems whose status is GLASS_BDSV_OK.  status_out: int32
 * [n_problems] or NULL.
 * workspace: NULL, or caller-owned device memory of at least
 * glass_bdsv_workspace_bytes(...) bytes aligned to the element size, where
 * the per-block-row factors [G_br | u_br] are kept for the back substitution.
 * Without it they are kept in on-chip memory, which limits how many problems
 * run at once and how long a chain can be; with it many more problems run
 * concurrently.  Its contents on entry do not matter; it must not be used by
 * another call at the same time.
 * Limits: state_size <= GLASS_BDSV_MAX_STATE_SIZE; without a workspace, one
 * problem's knot_points*state_size*(state_size+1) elements must fit in LDS
 * (GLASS_EUNSUPPORTED otherwise).
 */
size_t glass_bdsv_workspace_bytes(int state_size, int knot_points,
                                  int n_problems, glass_dtype dtype);
int glass_bdsv_batched(void* x, const void* S, const void* b, int state_size,
                       int knot_points, int n_problems, int* status_out,
                       void* workspace, size_t workspace_bytes,
                       glass_dtype dtype, void* hip_stream);

/*
 * Measurement aid, not a step of the solve: reads nbytes at src (device
 * memory, 16-byte aligned, nbytes a positive multiple of 16) once with
 * coalesced 16-byte non-temporal loads and writes, for each workgroup w
 * launched, sink[w] = the XOR of the 32-bit words that workgroup read.  The
 * XOR of sink[0 .. sink_words) (words past the workgroups launched are left
 * untouched, so zero them first) is the XOR of every 32-bit word of the
 * buffer.  At most sink_words workgroups are launched (8 per compute unit at
 * most); the time of the call gives the device's streaming-read rate, the
 * practical ceiling of the read-bound kernels above.
 */
int glass_stream_read(const void* src, size_t nbytes, unsigned* sink,
                      size_t sink_words, void* hip_stream);

/*
 * Measurement aid, not a step of the solve: the LDS read rate.  Launches up
 * to sink_words workgroups (8 per compute unit at most) of 256 threads; each
 * fills a 32 KB LDS buffer whose 32-bit word i is i * 0x9E3779B1 (mod 2^32),
 * then every thread t reads the 16-byte vectors (t + 256 u + 8 r) mod 2048
 * for r < rounds and u < 8 and folds their words into an XOR; sink[w] is the
 * XOR over workgroup w's threads (words past the workgroups launched are
 * left untouched).  bytes_per_load (4, 8 or 16) is what one LDS load
 * instruction reads per lane: each vector is read with one 16-byte load, two
 * 8-byte or four 4-byte ones; the XOR is the same.  *workgroups_out (host
 * memory) receives the number of workgroups launched, so the call reads
 * workgroups * 256 * rounds * 8 * 16 bytes from LDS.  rounds: 1 .. 2^20.
 */
int glass_lds_read(unsigned* sink, size_t sink_words, int rounds, int bytes_per_load,
                   int* workgroups_out, void* hip_stream);

/* Static text for a GLASS_* return code. */
const char* glass_status_string(int status);
/* Text describing the last failing call on this host thread ("" if none). */
const char* glass_last_error(void);
/* Library ABI version (major*10000 + minor*100 + patch).  0.2.0 added
 * glass_pcg_batched_pinned_rows and GLASS_PLACEMENT_S_RESIDENT; 0.3.0 added
 * glass_pcg_grid_noalloc; 0.4.0 added glass_pcg_batched_pinv_pass_rows; 0.5.0 added
 * glass_lds_read. */
int glass_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLASS_AMD_H */
