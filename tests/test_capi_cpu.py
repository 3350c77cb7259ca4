"""The C ABI library on the host: it loads, exports every declared symbol, and
rejects invalid arguments before touching a device (no GPU needed)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "glass_amd.h")
LIB = os.path.join(ROOT, "block_tridiagonal_pcg_bdmv_amd", "libglass_amd.so")

EINVAL, EUNSUPPORTED = -1, -2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(glass_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from block_tridiagonal_pcg_bdmv_amd import build
        build.build(verbose=False)
    import block_tridiagonal_pcg_bdmv_amd as glass
    return glass.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("glass_bdmv_batched", "glass_pcg_batched", "glass_pcg_grid",
                 "glass_pcg_batched_ex", "glass_pcg_grid_ex",
                 "glass_pcg_grid_workspace_bytes", "glass_status_string",
                 "glass_last_error", "glass_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.glass_status_string(0) == b"ok"
    assert lib.glass_status_string(-4).startswith(b"cooperative")
    assert lib.glass_version() >= 200


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: checks fail first


def _bdmv(lib, y=FAKE, S=FAKE, v=FAKE, ss=14, kp=64, B=1, dt=0):
    return lib.glass_bdmv_batched(y, S, v, ss, kp, B, dt, None)


def test_bdmv_argument_errors(lib):
    assert _bdmv(lib, y=None) == EINVAL
    assert _bdmv(lib, S=None) == EINVAL
    assert _bdmv(lib, v=ctypes.c_void_p(0x100002)) == EINVAL  # misaligned
    assert _bdmv(lib, ss=0) == EINVAL
    assert _bdmv(lib, kp=0) == EINVAL
    assert _bdmv(lib, B=-1) == EINVAL
    assert _bdmv(lib, dt=7) == EINVAL
    assert _bdmv(lib, ss=65) == EUNSUPPORTED
    assert b"state_size" in lib.glass_last_error()
    assert _bdmv(lib, B=0) == 0  # nothing to do, nothing launched


def _pcg(lib, x=FAKE, S=FAKE, P=FAKE, b=FAKE, ss=6, kp=32, B=1, it=20,
         rel=1e-6, ab=0.0, iters=FAKE, dt=0):
    return lib.glass_pcg_batched(x, S, P, b, ss, kp, B, it, rel, ab, iters, dt, None)


def test_pcg_argument_errors(lib):
    assert _pcg(lib, x=None) == EINVAL
    assert _pcg(lib, P=None) == EINVAL
    assert _pcg(lib, iters=None) == EINVAL
    assert _pcg(lib, it=-1) == EINVAL
    assert _pcg(lib, rel=-1.0) == EINVAL
    assert _pcg(lib, rel=float("nan")) == EINVAL
    assert _pcg(lib, ab=float("inf")) == EINVAL
    assert _pcg(lib, dt=2) == EINVAL
    assert _pcg(lib, ss=64, kp=200) == EUNSUPPORTED  # 12800 rows > 8192
    assert _pcg(lib, B=0) == 0


def test_grid_argument_errors_and_workspace_size(lib):
    ws = lib.glass_pcg_grid_workspace_bytes(12, 8192, 1)
    # Flag block, 8 copies of the tagged partials [2][G] in 64-byte slots,
    # tagged edges [2][G][4 ss][2 words]; G = kp/2 capped at 2048.
    assert ws == 256 + 8 * 2 * 2048 * 64 + 2 * 2048 * 4 * 12 * 2 * 8
    assert lib.glass_pcg_grid_workspace_bytes(12, 3, 1) == 0
    assert lib.glass_pcg_grid_workspace_bytes(0, 100, 1) == 0

    def grid(kp=8192, ws_ptr=ctypes.c_void_p(0x100000), ws_bytes=ws, it=10):
        return lib.glass_pcg_grid(FAKE, FAKE, FAKE, FAKE, 12, kp, it, 1e-10, 0.0,
                                  FAKE, ws_ptr, ws_bytes, 1, None)
    assert grid(kp=3) == EINVAL
    assert grid(ws_ptr=None) == EINVAL
    assert grid(ws_ptr=ctypes.c_void_p(0x100080)) == EINVAL  # not 256-aligned
    assert grid(ws_bytes=ws - 1) == EINVAL
    assert grid(it=-3) == EINVAL

    def grid_ex(flags):
        return lib.glass_pcg_grid_ex(FAKE, FAKE, FAKE, FAKE, 12, 8192, 10, 1e-10, 0.0,
                                     FAKE, None, None, ctypes.c_void_p(0x100000), ws, 1,
                                     flags, None)
    assert grid_ex(8) == EINVAL  # unknown flag bit
    assert grid_ex(1 | 2 | 16) == EINVAL
    assert grid_ex(0x80000000) == EINVAL


def test_bdsv_argument_errors(lib):
    def bdsv(x=FAKE, S=FAKE, b=FAKE, ss=14, kp=32, B=1, st=None, ws=None, wsb=0, dt=0):
        return lib.glass_bdsv_batched(x, S, b, ss, kp, B, st, ws, wsb, dt, None)
    assert bdsv(x=None) == EINVAL
    assert bdsv(S=None) == EINVAL
    assert bdsv(b=ctypes.c_void_p(0x100001)) == EINVAL
    assert bdsv(st=ctypes.c_void_p(0x100002)) == EINVAL
    assert bdsv(ss=0) == EINVAL
    assert bdsv(dt=3) == EINVAL
    assert bdsv(ss=25) == EUNSUPPORTED  # above GLASS_BDSV_MAX_STATE_SIZE
    assert bdsv(B=0) == 0
    need = lib.glass_bdsv_workspace_bytes(14, 32, 1, 0)
    assert need >= 32 * 14 * 15 * 4 and need % 256 == 0
    assert lib.glass_bdsv_workspace_bytes(25, 32, 1, 0) == 0
    assert bdsv(ws=FAKE, wsb=need - 1) == EINVAL  # too small
    assert bdsv(ws=ctypes.c_void_p(0x100002), wsb=need) == EINVAL  # misaligned


def test_placement_query_argument_errors(lib):
    assert lib.glass_pcg_batched_placement(0, 32, 0, 1, 0) == EINVAL
    assert lib.glass_pcg_batched_placement(6, 32, 5, 1, 0) == EINVAL
    assert lib.glass_pcg_batched_placement(64, 200, 0, 1, 0) == EUNSUPPORTED
    assert lib.glass_pcg_batched_placement(6, 32, 0, 1, 4) == EINVAL  # unknown flag
    assert lib.glass_pcg_batched_pinned_rows(0, 32, 0, 1, 0) == EINVAL
    assert lib.glass_pcg_batched_pinned_rows(6, 32, 5, 1, 0) == EINVAL
    assert lib.glass_pcg_batched_pinned_rows(64, 200, 0, 1, 0) == EUNSUPPORTED
    assert lib.glass_pcg_batched_pinned_rows(6, 32, 0, 1, 4) == EINVAL
    assert lib.glass_pcg_batched_pinv_pass_rows(0, 32, 0, 1, 0, 0) == EINVAL
    assert lib.glass_pcg_batched_pinv_pass_rows(6, 32, 5, 1, 0, 0) == EINVAL
    assert lib.glass_pcg_batched_pinv_pass_rows(64, 200, 0, 1, 0, 0) == EUNSUPPORTED
    assert lib.glass_pcg_batched_pinv_pass_rows(6, 32, 0, 1, 4, 0) == EINVAL
    assert lib.glass_pcg_batched_pinv_pass_rows(6, 32, 0, 1, 0, -1) == EINVAL


def test_pcg_ex_flag_errors(lib):
    def ex(flags):
        return lib.glass_pcg_batched_ex(FAKE, FAKE, FAKE, FAKE, 6, 32, 1, 20, 1e-6, 0.0, FAKE,
                                        None, None, 0, flags, None)
    assert ex(4) == EINVAL
    assert ex(0x80000000) == EINVAL
    assert ex(1 | 4) == EINVAL
    assert ex(2 | 8) == EINVAL


def test_grid_noalloc_argument_errors(lib):
    """glass_pcg_grid_noalloc runs the grid solve's checks (no workspace
    arguments) before anything touches a device."""
    def na(x=FAKE, kp=8192, it=10, rel=1e-10, flags=0, iters=FAKE, dt=1, st=None):
        return lib.glass_pcg_grid_noalloc(x, FAKE, FAKE, FAKE, 12, kp, it, rel, 0.0, iters,
                                          st, None, dt, flags, None)
    assert na(x=None) == EINVAL
    assert na(kp=3) == EINVAL
    assert na(it=-1) == EINVAL
    assert na(rel=float("nan")) == EINVAL
    assert na(iters=None) == EINVAL
    assert na(st=ctypes.c_void_p(0x100002)) == EINVAL
    assert na(dt=2) == EINVAL
    assert na(flags=8) == EINVAL
    assert b"flag" in lib.glass_last_error()
