"""The C-ABI library on the CPU: it loads, exports every entry point that
include/libscan.h declares, and rejects bad arguments on the host before any
HIP call (each call here is built to fail validation; none enqueues work)."""
import ctypes
import os
import re
import subprocess

import pytest

import prefix_scan_stream_amd as ps
from prefix_scan_stream_amd import build as psb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libscan.h")

INV, UNS, WS = ps.LS_ERR_INVALID_ARG, ps.LS_ERR_UNSUPPORTED, ps.LS_ERR_WORKSPACE
INT32, UINT32, F32 = 0, 1, 2
SUM, MAX, XOR, MIN, AND, OR, PROD, AFFINE = 0, 1, 2, 3, 4, 5, 6, 7


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ps.library_path()):
        psb.build()
    return ps.load_library()


def declared_functions():
    return psb.exported_symbols()


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("scan_inclusive", "scan_exclusive", "compact_if", "batched_row_scan",
                 "ls_scan_workspace_bytes", "ls_compact_workspace_bytes", "ls_status_string",
                 "ls_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ps.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else leaks out of the library
    assert exported == set(declared_functions())


def test_bounded_wait_test_library_exports_the_same_entry_points():
    """libscan_spin1.so (the same sources with waits that give up after one poll, for
    the GPU test of the error word) is built beside libscan.so with the same exports."""
    if not os.path.exists(psb.SPIN1_LIB):
        psb.build_bounded_wait_test_lib()
    out = subprocess.run(["nm", "-D", "--defined-only", psb.SPIN1_LIB], capture_output=True,
                         text=True, check=True).stdout
    assert set(re.findall(r" T (\w+)$", out, re.M)) == set(declared_functions())


def test_version_and_status_strings(lib):
    assert ps.ls_abi_version() == ps.ABI_VERSION == 5
    for s in range(6):
        assert ps.ls_status_string(s).startswith("LS_")
    assert "unknown" in ps.ls_status_string(99)


def test_workspace_queries(lib):
    b0 = ps.ls_scan_workspace_bytes(0, "int32", "sum")
    b1 = ps.ls_scan_workspace_bytes(1 << 28, "int32", "sum")
    assert b0 > 0 and b0 % 256 == 0 and b1 % 256 == 0
    # a 256-byte header plus one 256-byte status slot per tile of at least 8192 elements
    assert b0 < b1 <= 256 + 256 * ((1 << 28) // 8192) + 256
    c1 = ps.ls_compact_workspace_bytes(1 << 27, "int32")
    assert ps.ls_compact_workspace_bytes(0, "int32") < c1 <= 256 + 256 * ((1 << 27) // 8192) + 256
    sz = ctypes.c_size_t(0)
    assert lib.ls_scan_workspace_bytes(-1, INT32, SUM, ctypes.byref(sz)) == INV
    assert lib.ls_scan_workspace_bytes(10, 7, SUM, ctypes.byref(sz)) == INV
    assert lib.ls_scan_workspace_bytes(10, INT32, 9, ctypes.byref(sz)) == INV
    assert lib.ls_scan_workspace_bytes(10, F32, XOR, ctypes.byref(sz)) == UNS
    assert lib.ls_scan_workspace_bytes(10, INT32, SUM, None) == INV
    assert lib.ls_compact_workspace_bytes(-5, INT32, ctypes.byref(sz)) == INV


# Fake, never-dereferenced addresses: every call below must be rejected on the host.
A_IN = 0x7F0000000000
A_OUT = 0x7F0010000000
A_WS = 0x7F0020000000
A_TOT = 0x7F0030000000
BIG_WS = 1 << 30


def _scan(lib, fn, inp, out, n, t=INT32, op=SUM, total=None, ws=A_WS, wsb=BIG_WS):
    f = getattr(lib, fn)
    return f(inp, out, n, t, op, total, ws, wsb, None)


@pytest.mark.parametrize("fn", ["scan_inclusive", "scan_exclusive"])
def test_scan_validation(lib, fn):
    assert _scan(lib, fn, A_IN, A_OUT, -1) == INV                      # negative n
    assert _scan(lib, fn, None, A_OUT, 10) == INV                      # NULL input
    assert _scan(lib, fn, A_IN, None, 10) == INV                       # NULL output
    assert _scan(lib, fn, A_IN + 2, A_OUT, 10) == INV                  # misaligned
    assert _scan(lib, fn, A_IN, A_OUT + 1, 10) == INV
    assert _scan(lib, fn, A_IN, A_IN + 4, 10) == INV                   # partial overlap
    assert _scan(lib, fn, A_IN, A_OUT, 10, t=3) == INV                 # bad dtype
    assert _scan(lib, fn, A_IN, A_OUT, 10, op=8) == INV                # bad op
    assert _scan(lib, fn, A_IN, A_OUT, 10, op=-1) == INV
    assert _scan(lib, fn, A_IN, A_OUT, 10, t=F32, op=XOR) == UNS       # float xor
    for op in (AND, OR, AFFINE):                                        # other bitwise / maps on floats
        assert _scan(lib, fn, A_IN, A_OUT, 10, t=F32, op=op) == UNS
    assert _scan(lib, fn, A_IN, A_OUT, 10, t=INT32, op=AFFINE) == UNS  # affine maps are uint32
    for t, op in ((F32, MIN), (F32, PROD), (INT32, PROD), (UINT32, AFFINE), (INT32, AND)):
        assert _scan(lib, fn, A_IN, A_OUT, 10, t=t, op=op, ws=None) == WS  # defined: reaches the ws check
    assert _scan(lib, fn, A_IN, A_OUT, 10, ws=None) == WS              # no workspace
    assert _scan(lib, fn, A_IN, A_OUT, 1 << 20, wsb=64) == WS          # workspace too small
    assert _scan(lib, fn, A_IN, A_OUT, 10, ws=A_WS + 8) == INV         # workspace misaligned
    assert _scan(lib, fn, A_IN, A_OUT, 1000, ws=A_OUT + 16) == INV     # workspace overlaps out
    assert _scan(lib, fn, A_IN, A_OUT, 10, total=A_OUT + 8) == INV     # total inside out
    assert _scan(lib, fn, A_IN, A_OUT, 10, total=A_TOT + 2) == INV     # total misaligned
    # error precedence: invalid argument before unsupported before workspace
    assert _scan(lib, fn, None, A_OUT, 10, t=F32, op=XOR, ws=None) == INV
    assert _scan(lib, fn, A_IN, A_OUT, 10, t=F32, op=XOR, ws=None) == UNS


def test_workspace_init_and_check_validation(lib):
    """Both reject a bad workspace on the host, before any HIP call."""
    init, check = lib.ls_workspace_init, lib.ls_workspace_check
    assert init(None, 4096, None) == INV
    assert init(A_WS + 8, 4096, None) == INV      # misaligned
    assert init(A_WS, 4100, None) == INV          # not a multiple of 16
    assert init(A_WS, 128, None) == INV           # smaller than the 256-byte header
    flags = ctypes.c_uint32(7)
    assert check(None, ctypes.byref(flags), None) == INV
    assert check(A_WS + 4, ctypes.byref(flags), None) == INV
    assert flags.value == 7                        # untouched on error
    assert ps.ls_status_string(ps.LS_ERR_INCOMPLETE).startswith("LS_ERR_INCOMPLETE")


def test_size_limits(lib):
    """Scans take at most 2^40 elements (32-bit tile ids), compactions 2^36 - 1
    (36-bit counts); larger sizes are invalid arguments."""
    sz = ctypes.c_size_t(0)
    assert lib.ls_scan_workspace_bytes(1 << 40, INT32, SUM, ctypes.byref(sz)) == 0
    assert lib.ls_scan_workspace_bytes((1 << 40) + 1, INT32, SUM, ctypes.byref(sz)) == INV
    assert lib.ls_segmented_workspace_bytes((1 << 40) + 1, INT32, SUM, ctypes.byref(sz)) == INV
    assert lib.ls_compact_workspace_bytes((1 << 36) - 1, INT32, ctypes.byref(sz)) == 0
    assert lib.ls_compact_workspace_bytes(1 << 36, INT32, ctypes.byref(sz)) == INV
    far = A_IN - (1 << 44)
    assert lib.compact_if(A_IN, far, A_TOT, 1 << 36, INT32, 0, 0, A_WS, BIG_WS, None) == INV
    assert _scan(lib, "scan_inclusive", A_IN, far, (1 << 40) + 1) == INV


def test_noalloc_scan_validation(lib):
    """scan_noalloc checks its arguments like the scans (on the host, before the
    library's fixed workspace is looked up) and refuses n above its maximum."""
    f = lib.scan_noalloc
    assert f(A_IN, A_OUT, -1, INT32, SUM, 1, None, None) == INV
    assert f(None, A_OUT, 10, INT32, SUM, 1, None, None) == INV
    assert f(A_IN, A_OUT + 2, 10, INT32, SUM, 0, None, None) == INV
    assert f(A_IN, A_IN + 4, 10, INT32, SUM, 0, None, None) == INV
    assert f(A_IN, A_OUT, 10, 3, SUM, 0, None, None) == INV
    assert f(A_IN, A_OUT, 10, F32, XOR, 0, None, None) == UNS
    assert f(A_IN, A_OUT, 10, INT32, SUM, 0, A_OUT + 8, None) == INV
    far = A_IN - (1 << 40)  # far enough below `in` that the large sizes do not overlap it
    assert f(A_IN, far, ps.SCAN_NOALLOC_MAX_N + 1, INT32, SUM, 1, None, None) == WS
    assert f(A_IN, far, 1 << 36, F32, MAX, 0, None, None) == WS
    # the fixed 8 MiB workspace holds the single pass's status words at the maximum n
    for t, op in ((INT32, SUM), (F32, SUM), (UINT32, AFFINE)):
        need = ctypes.c_size_t(0)
        assert lib.ls_scan_workspace_bytes(ps.SCAN_NOALLOC_MAX_N, t, op, ctypes.byref(need)) == 0
        assert need.value <= 8 << 20


def test_extended_entry_points_validation(lib):
    sz = ctypes.c_size_t(0)
    for scheme in range(4):
        assert lib.ls_scan_ex_workspace_bytes(1 << 20, INT32, SUM, scheme, ctypes.byref(sz)) == 0
        assert sz.value > 0
    single = ctypes.c_size_t(0)
    lib.ls_scan_ex_workspace_bytes(1 << 20, F32, SUM, 0, ctypes.byref(single))
    lib.ls_scan_ex_workspace_bytes(1 << 20, F32, SUM, 3, ctypes.byref(sz))
    # a 256-byte header and one 256-byte status slot per tile of the smallest tile:
    # 16384 elements for the single pass (the affine maps'), 32768 for the
    # deterministic one
    assert single.value == 256 + 256 * -(-(1 << 20) // 16384)
    assert sz.value == 256 + 256 * -(-(1 << 20) // 32768)
    assert lib.ls_scan_ex_workspace_bytes(1 << 20, INT32, SUM, 4, ctypes.byref(sz)) == INV
    assert lib.ls_scan_ex_workspace_bytes(10, F32, XOR, 1, ctypes.byref(sz)) == UNS
    # three-phase workspaces grow with the recursion over the tile totals
    assert ps.ls_scan_ex_workspace_bytes(1 << 34, "int32", "sum", "reduce_then_scan") > \
        2 * 4 * ((1 << 34) // (1 << 14))

    def sx(scheme=0, n=10, ws=A_WS, wsb=BIG_WS, t=INT32, op=SUM, excl=1):
        return lib.scan_ex(A_IN, A_OUT, n, t, op, excl, scheme, None, ws, wsb, None)

    assert sx(scheme=4) == INV
    assert sx(scheme=3, ws=None) == WS  # the deterministic single pass is a valid scheme
    assert sx(scheme=-1) == INV
    assert sx(scheme=1, n=-2) == INV
    assert sx(scheme=2, t=F32, op=XOR) == UNS
    assert sx(scheme=1, ws=None) == WS
    assert sx(scheme=2, n=1 << 24, wsb=256) == WS

    def bx(kind=0, rows=4, cols=100):
        return lib.batched_row_scan_ex(A_IN, A_OUT, rows, cols, INT32, SUM, 1, kind, None)

    assert bx(kind=4) == INV
    assert bx(kind=-1) == INV
    assert bx(kind=3, rows=-1) == INV
    assert lib.batched_row_scan_ex(None, None, 0, 5, INT32, SUM, 1, 2, None) == ps.LS_OK


def test_radix_sort_validation(lib):
    A_V1, A_V2 = 0x7F0040000000, 0x7F0050000000
    sz = ctypes.c_size_t(0)
    assert lib.ls_radix_sort_workspace_bytes(1 << 20, UINT32, 1, ctypes.byref(sz)) == 0
    with_v = sz.value
    assert lib.ls_radix_sort_workspace_bytes(1 << 20, UINT32, 0, ctypes.byref(sz)) == 0
    assert with_v > sz.value > 0
    assert lib.ls_radix_sort_workspace_bytes(-1, UINT32, 0, ctypes.byref(sz)) == INV
    assert lib.ls_radix_sort_workspace_bytes(1 << 32, UINT32, 0, ctypes.byref(sz)) == INV
    assert lib.ls_radix_sort_workspace_bytes(10, 5, 0, ctypes.byref(sz)) == INV

    def rs(ki=A_IN, ko=A_OUT, vi=None, vo=None, n=100, t=UINT32, ws=A_WS, wsb=BIG_WS):
        return lib.radix_sort(ki, ko, vi, vo, n, t, ws, wsb, None)

    assert rs(n=-1) == INV
    assert rs(n=1 << 32) == INV
    assert rs(t=7) == INV
    assert rs(vi=A_V1) == INV            # values in without values out
    assert rs(vo=A_V2) == INV
    assert rs(ki=None) == INV
    assert rs(ko=A_IN + 8) == INV        # partial overlap of keys
    assert rs(vi=A_V1, vo=A_IN) == INV   # values overlap keys
    assert rs(ws=None) == WS
    assert rs(n=1 << 20, wsb=4096) == WS
    assert rs(ws=A_WS + 4) == INV        # workspace alignment


def test_compact_validation(lib):
    def call(inp=A_IN, out=A_OUT, count=A_TOT, n=10, t=INT32, cmp=0, ws=A_WS, wsb=BIG_WS):
        return lib.compact_if(inp, out, count, n, t, cmp, 5, ws, wsb, None)

    assert call(n=-1) == INV
    assert call(count=None) == INV
    assert call(count=A_TOT + 4) == INV         # count must be 8-byte aligned
    assert call(inp=None) == INV
    assert call(out=A_IN) == INV                # compaction never runs in place
    assert call(out=A_IN + 16) == INV
    assert call(cmp=6) == INV
    assert call(t=9) == INV
    assert call(count=A_OUT + 8) == INV         # count inside out
    assert call(ws=None) == WS
    assert call(n=1 << 20, wsb=256) == WS


def test_flags_and_indices_validation(lib):
    A_F = 0x7F0060000000

    def cf(inp=A_IN, flags=A_F, out=A_OUT, count=A_TOT, n=10, ws=A_WS, wsb=BIG_WS):
        return lib.compact_flags(inp, flags, out, count, n, ws, wsb, None)

    assert cf(n=-1) == INV
    assert cf(flags=None) == INV
    assert cf(inp=None) == INV
    assert cf(out=A_IN) == INV
    assert cf(flags=A_OUT + 3) == INV          # flags overlap out
    assert cf(count=None) == INV
    assert cf(ws=None) == WS
    assert cf(flags=A_F + 1, ws=None) == WS    # any flag alignment is accepted

    def si(inp=A_IN, out=A_OUT, n=10, t=INT32, cmp=0):
        return lib.select_indices_if(inp, out, A_TOT, n, t, cmp, 0, A_WS, BIG_WS, None)

    assert si(n=1 << 32) == INV                # indices are uint32
    assert si(cmp=9) == INV
    assert si(inp=None) == INV
    assert lib.select_indices_flags(None, A_OUT, A_TOT, 10, A_WS, BIG_WS, None) == INV
    assert lib.select_indices_flags(A_F, A_OUT, A_TOT, 1 << 32, A_WS, BIG_WS, None) == INV
    assert lib.select_indices_flags(A_F, A_OUT, A_TOT, 10, None, 0, None) == WS


def test_segmented_validation(lib):
    A_H = 0x7F0070000000

    def sg(inp=A_IN, out=A_OUT, n=10, t=INT32, op=SUM, heads=A_H, total=None, ws=A_WS, wsb=BIG_WS):
        return lib.segmented_scan(inp, out, n, t, op, 0, heads, total, ws, wsb, None)

    def so(inp=A_IN, out=A_OUT, n=10, t=INT32, op=SUM, offs=A_H, nseg=3, ws=A_WS, wsb=BIG_WS):
        return lib.segmented_scan_offsets(inp, out, n, t, op, 1, offs, nseg, None, ws, wsb, None)

    assert sg(n=-1) == INV
    assert sg(heads=None) == INV
    assert sg(inp=None) == INV
    assert sg(out=A_IN + 4) == INV                 # partial overlap
    assert sg(heads=A_OUT + 5) == INV              # heads inside out
    assert sg(op=8) == INV
    assert sg(t=F32, op=XOR) == UNS
    assert sg(t=INT32, op=AFFINE) == UNS
    assert sg(ws=None) == WS
    assert sg(heads=A_H + 1, ws=None) == WS        # any heads alignment
    assert sg(out=A_IN, ws=None) == WS             # in place is allowed
    assert sg(total=A_OUT + 8) == INV
    assert so(nseg=0) == INV                        # n > 0 needs a segment
    assert so(offs=None) == INV
    assert so(offs=A_H + 4) == INV                  # offsets 8-byte aligned
    assert so(offs=A_OUT) == INV                    # offsets inside out
    assert so(ws=None) == WS
    assert so(n=0, inp=None, out=None, offs=None, nseg=0, ws=None) == WS
    # empty and no total: valid, and nothing is enqueued
    assert so(n=0, inp=None, out=None, offs=None, nseg=0) == ps.LS_OK
    assert sg(n=0, inp=None, out=None, heads=None) == ps.LS_OK
    sz = ctypes.c_size_t(0)
    assert lib.ls_segmented_workspace_bytes(1 << 20, INT32, SUM, ctypes.byref(sz)) == 0 and sz.value > 0
    assert lib.ls_segmented_workspace_bytes(10, F32, AND, ctypes.byref(sz)) == UNS


def test_batched_validation(lib):
    def call(inp=A_IN, out=A_OUT, rows=4, cols=64, t=F32, op=SUM, excl=1):
        return lib.batched_row_scan(inp, out, rows, cols, t, op, excl, None)

    assert call(rows=-1) == INV
    assert call(cols=-1) == INV
    assert call(inp=None) == INV
    assert call(out=A_IN + 4) == INV
    assert call(t=F32, op=XOR) == UNS
    assert call(t=F32, op=AFFINE) == UNS
    assert call(t=INT32, op=AFFINE) == UNS
    assert call(op=8) == INV
    assert call(rows=1 << 40, cols=1 << 40) == INV  # size overflow
    # empty shapes are a no-op even with NULL pointers (nothing is enqueued)
    assert call(inp=None, out=None, rows=0) == ps.LS_OK
    assert call(inp=None, out=None, cols=0) == ps.LS_OK


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError):
        ps.scan_exclusive(x)
    with pytest.raises(ValueError):
        ps.compact_if(x, "lt", 3)
    with pytest.raises(ValueError):
        ps.batched_row_scan(x.reshape(2, 4))
