"""Python binding of the glass_amd C ABI (include/glass_amd.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream, ctypes passes raw pointers, and every step runs in the HIP kernels of
``libglass_amd.so``.  There is no CPU or PyTorch fallback -- if the library is
missing, every call raises.

Because the C ABI takes raw pointers, this layer checks each tensor's device,
dtype, contiguity and element count against the sizes implied by
``state_size`` / ``knot_points`` before anything is launched.
"""

from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "GlassError", "load", "library_path", "bdmv_batched", "pcg_batched",
    "pcg_grid", "pcg_grid_workspace_bytes", "pcg_grid_noalloc", "bdsv_batched", "bdsv_workspace_bytes",
    "CONVERGED",
    "MAX_ITERS", "BREAKDOWN", "GRID_TIMEOUT", "BDSV_OK", "BDSV_NOT_SPD", "GRID_EXCLUSIVE",
    "PCG_PINV_BLOCK_DIAGONAL", "PCG_PINV_DIAGONAL_BLOCKS", "GRID_SINGLE_REDUCTION",
    "GRID_KEEP_WORKSPACE",
    "pcg_batched_placement", "pcg_batched_pinned_rows", "PLACEMENT_RESIDENT",
    "PLACEMENT_STREAMED_PREFETCH",
    "PLACEMENT_STREAMED", "PLACEMENT_S_RESIDENT", "PLACEMENT_SEVERAL_PER_WAVE", "stream_read",
    "pcg_batched_pinv_pass_rows", "lds_read",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# GLASS_AMD_LIBRARY points at another build of the same library (for A/B
# timing of build options); the default is the in-tree build.
_LIB_PATH = os.environ.get("GLASS_AMD_LIBRARY") or os.path.join(_HERE, "libglass_amd.so")
_lib = None
_lock = threading.Lock()

GLASS_F32, GLASS_F64 = 0, 1
CONVERGED, MAX_ITERS, BREAKDOWN, GRID_TIMEOUT = 0, 1, 2, 3
BDSV_OK, BDSV_NOT_SPD = 0, 1
GRID_EXCLUSIVE = 1  # glass_pcg_grid_ex flag: ordinary dispatch on the stream's queue
GRID_SINGLE_REDUCTION = 2  # glass_pcg_grid_ex flag: one grid reduction per iteration
GRID_KEEP_WORKSPACE = 4  # glass_pcg_grid_ex flag: the workspace is kept for grid solves
PCG_PINV_BLOCK_DIAGONAL = 1  # glass_pcg_batched_ex flag: Pinv's L and R blocks are zero
PCG_PINV_DIAGONAL_BLOCKS = 2  # glass_pcg_batched_ex flag: Pinv is packed D blocks [B, kp, ss, ss]


class GlassError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__("%s failed with %d: %s" % (where, code, detail))
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load ``libglass_amd.so`` (built by ``build.py``); raises if absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "libglass_amd.so is not built (run __graft_entry__.build() or "
                "python block_tridiagonal_pcg_bdmv_amd/build.py)")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, D, Z, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_size_t, ctypes.c_uint
        sigs = {
            "glass_bdmv_batched": ([P, P, P, I, I, I, I, P], I),
            "glass_pcg_batched": ([P, P, P, P, I, I, I, I, D, D, P, I, P], I),
            "glass_pcg_batched_ex": ([P, P, P, P, I, I, I, I, D, D, P, P, P, I, U, P], I),
            "glass_bdsv_batched": ([P, P, P, I, I, I, P, P, Z, I, P], I),
            "glass_bdsv_workspace_bytes": ([I, I, I, I], Z),
            "glass_pcg_batched_placement": ([I, I, I, I, U], I),
            "glass_pcg_batched_pinned_rows": ([I, I, I, I, U], I),
            "glass_pcg_batched_pinv_pass_rows": ([I, I, I, I, U, I], I),
            "glass_pcg_grid_workspace_bytes": ([I, I, I], Z),
            "glass_pcg_grid": ([P, P, P, P, I, I, I, D, D, P, P, Z, I, P], I),
            "glass_pcg_grid_ex": ([P, P, P, P, I, I, I, D, D, P, P, P, P, Z, I, U, P], I),
            "glass_pcg_grid_noalloc": ([P, P, P, P, I, I, I, D, D, P, P, P, I, U, P], I),
            "glass_stream_read": ([P, Z, P, Z, P], I),
            "glass_lds_read": ([P, Z, I, I, ctypes.POINTER(ctypes.c_int), P], I),
            "glass_status_string": ([I], ctypes.c_char_p),
            "glass_last_error": ([], ctypes.c_char_p),
            "glass_version": ([], I),
        }
        for name, (args, res) in sigs.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
        return lib


def _check(rc: int, where: str):
    if rc != 0:
        lib = load()
        raise GlassError(rc, where, "%s (%s)" % (
            lib.glass_status_string(rc).decode(), lib.glass_last_error().decode()))


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return GLASS_F32
    if t.dtype == torch.float64:
        return GLASS_F64
    raise TypeError("tensors must be float32 or float64, got %s" % t.dtype)


def _dev(t, name, numel, dtype=None):
    """Raw device pointer of ``t`` once it is a contiguous device tensor of
    ``numel`` elements (and ``dtype``); raises otherwise."""
    try:
        if (t.is_cuda and t.is_contiguous() and t.numel() == numel
                and (dtype is None or t.dtype == dtype)):
            return t.data_ptr()
    except AttributeError:
        raise TypeError("%s must be a torch tensor" % name) from None
    _dev_fail(t, name, numel, dtype)


def _dev_fail(t, name, numel, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))


def _stream(stream):
    """The raw HIP stream: ``stream``'s, or torch's current stream on the
    current device (read without building a Stream object when torch offers
    that)."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _problems(S, ss, kp):
    per = kp * ss * 3 * ss
    if ss < 1 or kp < 1 or S.numel() % per != 0:
        raise ValueError("S size is not a multiple of knot_points*state_size*3*state_size")
    return S.numel() // per


def bdmv_batched(y, S, v, state_size: int, knot_points: int, stream=None):
    """y = A_bd v for every problem (page "Block-tridiagonal Solves", section
    "Matvec -- glass::bdmv").  y, v: padded [B, (kp+2)*ss]; only the interior
    of y is written."""
    ss, kp = int(state_size), int(knot_points)
    B = _problems(S, ss, kp)
    dt = S.dtype
    vec = (kp + 2) * ss * B
    args = (_dev(y, "y", vec, dt), _dev(S, "S", S.numel(), dt), _dev(v, "v", vec, dt))
    rc = load().glass_bdmv_batched(*args, ss, kp, B, _dtype_code(S), _stream(stream))
    _check(rc, "glass_bdmv_batched")


def pcg_batched(x, S, Pinv, b, state_size: int, knot_points: int, max_iters: int,
                rel_tol: float, abs_tol: float, iters_out, status_out=None,
                rho_out=None, stream=None, pinv_block_diagonal=False,
                pinv_diagonal_blocks=False):
    """Batched PCG (page "Block-tridiagonal Solves", section "Solve --
    glass::pcg").  x: [B, kp*ss] initial guess in, solution out; iters_out
    (and status_out) int32 [B]; rho_out dtype [B, 2].
    ``pinv_block_diagonal=True`` passes GLASS_PCG_PINV_BLOCK_DIAGONAL: the
    caller asserts that Pinv's L and R blocks are zero.
    ``pinv_diagonal_blocks=True`` passes GLASS_PCG_PINV_DIAGONAL_BLOCKS: Pinv
    holds only the D blocks, packed as [B, kp, ss, ss]."""
    import torch
    ss, kp = int(state_size), int(knot_points)
    B = _problems(S, ss, kp)
    dt = S.dtype
    n = kp * ss
    p_numel = B * n * ss if pinv_diagonal_blocks else S.numel()
    a = (_dev(x, "x", B * n, dt), _dev(S, "S", S.numel(), dt),
         _dev(Pinv, "Pinv", p_numel, dt), _dev(b, "b", B * n, dt))
    flags = (PCG_PINV_BLOCK_DIAGONAL if pinv_block_diagonal else 0) | \
        (PCG_PINV_DIAGONAL_BLOCKS if pinv_diagonal_blocks else 0)
    it = _dev(iters_out, "iters_out", B, torch.int32)
    st = _dev(status_out, "status_out", B, torch.int32) if status_out is not None else None
    rh = _dev(rho_out, "rho_out", 2 * B, dt) if rho_out is not None else None
    rc = load().glass_pcg_batched_ex(*a, ss, kp, B, int(max_iters), float(rel_tol),
                                     float(abs_tol), it, st, rh, _dtype_code(S),
                                     flags, _stream(stream))
    _check(rc, "glass_pcg_batched_ex")


def bdsv_workspace_bytes(state_size: int, knot_points: int, n_problems: int, dtype) -> int:
    import torch
    code = GLASS_F32 if dtype == torch.float32 else GLASS_F64
    return int(load().glass_bdsv_workspace_bytes(int(state_size), int(knot_points),
                                                 int(n_problems), code))


def bdsv_batched(x, S, b, state_size: int, knot_points: int, status_out=None,
                 workspace=None, stream=None):
    """Direct solve S x = b per problem (page "Block-tridiagonal Solves",
    glass::bdsv).  x, b: [B, kp*ss]; status_out int32 [B] (BDSV_OK or
    BDSV_NOT_SPD; x is written only where it is BDSV_OK); workspace: None or
    a contiguous device tensor of at least ``bdsv_workspace_bytes`` bytes."""
    import torch
    ss, kp = int(state_size), int(knot_points)
    B = _problems(S, ss, kp)
    dt = S.dtype
    n = kp * ss
    a = (_dev(x, "x", B * n, dt), _dev(S, "S", S.numel(), dt), _dev(b, "b", B * n, dt))
    st = _dev(status_out, "status_out", B, torch.int32) if status_out is not None else None
    if workspace is None:
        wp, wb = None, 0
    else:
        if not (workspace.is_cuda and workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous device tensor")
        wp, wb = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    rc = load().glass_bdsv_batched(*a, ss, kp, B, st, wp, wb, _dtype_code(S), _stream(stream))
    _check(rc, "glass_bdsv_batched")


PLACEMENT_RESIDENT, PLACEMENT_STREAMED_PREFETCH, PLACEMENT_STREAMED, PLACEMENT_S_RESIDENT = 0, 1, 2, 3
PLACEMENT_SEVERAL_PER_WAVE = 4


def pcg_batched_placement(state_size: int, knot_points: int, dtype, aligned16=True,
                          pinv_block_diagonal=False, pinv_diagonal_blocks=False) -> int:
    """Where pcg_batched keeps S and Pinv on the current device for this shape:
    PLACEMENT_RESIDENT (read once per solve), PLACEMENT_STREAMED[_PREFETCH]
    (read once per matvec pass) or PLACEMENT_S_RESIDENT (S read once, Pinv once
    per pass).  Raises for shapes the solve rejects."""
    import torch
    code = GLASS_F32 if dtype == torch.float32 else GLASS_F64
    rc = load().glass_pcg_batched_placement(int(state_size), int(knot_points), code,
                                            1 if aligned16 else 0,
                                            (PCG_PINV_BLOCK_DIAGONAL if pinv_block_diagonal else 0)
                                            | (PCG_PINV_DIAGONAL_BLOCKS
                                               if pinv_diagonal_blocks else 0))
    if rc < 0:
        _check(rc, "glass_pcg_batched_placement")
    return rc


def pcg_batched_pinv_pass_rows(state_size: int, knot_points: int, dtype, pass_index: int,
                               aligned16=True, pinv_block_diagonal=False,
                               pinv_diagonal_blocks=False) -> int:
    """Pinv rows per problem that matvec pass ``pass_index`` of pcg_batched
    reads from memory on the current device (pass 0: z = Pinv r0, with the
    rows kept on chip for the whole solve; pass p >= 1: iteration p).  Raises
    for shapes the solve rejects."""
    import torch
    code = GLASS_F32 if dtype == torch.float32 else GLASS_F64
    rc = load().glass_pcg_batched_pinv_pass_rows(
        int(state_size), int(knot_points), code, 1 if aligned16 else 0,
        (PCG_PINV_BLOCK_DIAGONAL if pinv_block_diagonal else 0)
        | (PCG_PINV_DIAGONAL_BLOCKS if pinv_diagonal_blocks else 0), int(pass_index))
    if rc < 0:
        _check(rc, "glass_pcg_batched_pinv_pass_rows")
    return rc


def pcg_batched_pinned_rows(state_size: int, knot_points: int, dtype, aligned16=True,
                            pinv_block_diagonal=False, pinv_diagonal_blocks=False) -> int:
    """Pinv rows per problem that the S-resident placement keeps in LDS for the
    whole solve (read once; the others are read once per matvec pass); 0 for
    the other placements.  Raises for shapes the solve rejects."""
    import torch
    code = GLASS_F32 if dtype == torch.float32 else GLASS_F64
    rc = load().glass_pcg_batched_pinned_rows(int(state_size), int(knot_points), code,
                                              1 if aligned16 else 0,
                                              (PCG_PINV_BLOCK_DIAGONAL if pinv_block_diagonal else 0)
                                              | (PCG_PINV_DIAGONAL_BLOCKS
                                                 if pinv_diagonal_blocks else 0))
    if rc < 0:
        _check(rc, "glass_pcg_batched_pinned_rows")
    return rc


def pcg_grid_workspace_bytes(state_size: int, knot_points: int, dtype) -> int:
    import torch
    code = GLASS_F32 if dtype == torch.float32 else GLASS_F64
    return int(load().glass_pcg_grid_workspace_bytes(int(state_size), int(knot_points), code))


def pcg_grid(x, S, Pinv, b, state_size: int, knot_points: int, max_iters: int,
             rel_tol: float, abs_tol: float, iters_out, workspace,
             status_out=None, rho_out=None, stream=None, exclusive=False,
             single_reduction=False, keep_workspace=False):
    """One PCG solve over a cooperative grid.  Same arguments as
    ``pcg_batched`` with one problem, plus a device ``workspace`` tensor of at
    least ``pcg_grid_workspace_bytes`` bytes (any dtype, 256-byte aligned).
    ``exclusive=True`` passes GLASS_GRID_EXCLUSIVE: an ordinary dispatch on
    the stream's queue, for callers that know no other kernel occupies the
    device during the solve.  ``single_reduction=True`` passes
    GLASS_GRID_SINGLE_REDUCTION: the single-reduction form of PCG (one grid
    reduction per iteration; same iterates in exact arithmetic).
    ``keep_workspace=True`` passes GLASS_GRID_KEEP_WORKSPACE: the workspace
    is used by nothing but grid solves between calls, so its exchange words
    need no clearing per solve."""
    import torch
    ss, kp = int(state_size), int(knot_points)
    if _problems(S, ss, kp) != 1:
        raise ValueError("pcg_grid solves exactly one problem")
    dt = S.dtype
    n = kp * ss
    a = (_dev(x, "x", n, dt), _dev(S, "S", S.numel(), dt),
         _dev(Pinv, "Pinv", S.numel(), dt), _dev(b, "b", n, dt))
    it = _dev(iters_out, "iters_out", 1, torch.int32)
    st = _dev(status_out, "status_out", 1, torch.int32) if status_out is not None else None
    rh = _dev(rho_out, "rho_out", 2, dt) if rho_out is not None else None
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    wbytes = workspace.numel() * workspace.element_size()
    rc = load().glass_pcg_grid_ex(*a, ss, kp, int(max_iters), float(rel_tol),
                                  float(abs_tol), it, st, rh,
                                  ctypes.c_void_p(workspace.data_ptr()), wbytes,
                                  _dtype_code(S),
                                  (GRID_EXCLUSIVE if exclusive else 0)
                                  | (GRID_SINGLE_REDUCTION if single_reduction else 0)
                                  | (GRID_KEEP_WORKSPACE if keep_workspace else 0),
                                  _stream(stream))
    _check(rc, "glass_pcg_grid_ex")


def pcg_grid_noalloc(x, S, Pinv, b, state_size: int, knot_points: int, max_iters: int,
                     rel_tol: float, abs_tol: float, iters_out, status_out=None,
                     rho_out=None, stream=None, exclusive=False, single_reduction=False):
    """``pcg_grid`` without a workspace (glass_pcg_grid_noalloc): the
    exchange area is the library's static per-device scratch, so the call
    allocates nothing.  Calls that overlap in time on one device race."""
    import torch
    ss, kp = int(state_size), int(knot_points)
    if _problems(S, ss, kp) != 1:
        raise ValueError("pcg_grid_noalloc solves exactly one problem")
    dt = S.dtype
    n = kp * ss
    a = (_dev(x, "x", n, dt), _dev(S, "S", S.numel(), dt),
         _dev(Pinv, "Pinv", S.numel(), dt), _dev(b, "b", n, dt))
    it = _dev(iters_out, "iters_out", 1, torch.int32)
    st = _dev(status_out, "status_out", 1, torch.int32) if status_out is not None else None
    rh = _dev(rho_out, "rho_out", 2, dt) if rho_out is not None else None
    rc = load().glass_pcg_grid_noalloc(*a, ss, kp, int(max_iters), float(rel_tol),
                                       float(abs_tol), it, st, rh, _dtype_code(S),
                                       (GRID_EXCLUSIVE if exclusive else 0)
                                       | (GRID_SINGLE_REDUCTION if single_reduction else 0),
                                       _stream(stream))
    _check(rc, "glass_pcg_grid_noalloc")


def lds_read(sink, rounds: int, bytes_per_load: int = 16, stream=None) -> int:
    """Measurement aid (glass_lds_read): every workgroup launched fills 32 KB
    of LDS and its threads read it back ``rounds`` * 8 times as 16-byte
    vectors, each with loads of ``bytes_per_load`` (4, 8 or 16) bytes per lane;
    ``sink`` (int32 device tensor, zeroed by the caller) receives one XOR per
    workgroup.  Returns the number of workgroups launched."""
    import torch
    sk = _dev(sink, "sink", sink.numel(), torch.int32)
    wg = ctypes.c_int(0)
    rc = load().glass_lds_read(sk, sink.numel(), int(rounds), int(bytes_per_load),
                               ctypes.byref(wg), _stream(stream))
    _check(rc, "glass_lds_read")
    return wg.value


def stream_read(src, sink, stream=None):
    """Measurement aid (glass_stream_read): read every byte of the contiguous
    device tensor ``src`` once; ``sink`` (int32 device tensor, zeroed by the
    caller) receives one XOR of 32-bit words per workgroup launched."""
    import torch
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    sk = _dev(sink, "sink", sink.numel(), torch.int32)
    rc = load().glass_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, sk, sink.numel(),
                                  _stream(stream))
    _check(rc, "glass_stream_read")
