"""Bounded waits end with a report, not a hang.

Every wait of one tile on another (the chased prefixes and the decoupled look-back
of the scans, compaction and segmented scans) gives up after a fixed number of empty
polls and sets bit 0 of the workspace error word.  prefix_scan_stream_amd/libscan_spin1.so
(built by build() from the same sources) gives up after a single empty poll, so in
a multi-tile call some tile is certain to give up.  Each call must still complete
and must report it; its outputs are then unspecified.

Only entry points whose stores stay inside their buffers whatever a tile's offset
are called here: scan tiles write through their own byte range, and compaction's
offsets combine only non-negative counts, so a prefix cut short is never larger than
the true one.  The radix sort is left out: its scatter addresses come from its scan."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "prefix_scan_stream_amd", "libscan_spin1.so")
INT32, SUM, LT, DETERMINISTIC = 0, 0, 0, 3
N = 1 << 25  # hundreds of tiles for every kernel below


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB)
    vp, i64, u32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int, ctypes.c_size_t
    szp = ctypes.POINTER(ctypes.c_size_t)
    L.ls_scan_workspace_bytes.argtypes = [i64, i32, i32, szp]
    L.ls_scan_ex_workspace_bytes.argtypes = [i64, i32, i32, i32, szp]
    L.ls_compact_workspace_bytes.argtypes = [i64, i32, szp]
    L.ls_segmented_workspace_bytes.argtypes = [i64, i32, i32, szp]
    L.scan_exclusive.argtypes = [vp, vp, i64, i32, i32, vp, vp, sz, vp]
    L.scan_ex.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp]
    L.compact_if.argtypes = [vp, vp, vp, i64, i32, i32, u32, vp, sz, vp]
    L.segmented_scan.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp, sz, vp]
    return L


def workspace(query, *args):
    nbytes = ctypes.c_size_t(0)
    assert query(*args, ctypes.byref(nbytes)) == 0
    return torch.empty(nbytes.value, dtype=torch.uint8, device=DEV)


def error_word(ws):
    torch.cuda.synchronize()  # returns only if every kernel of the call has ended
    return int(ws[4:8].cpu().numpy().view(np.uint32)[0])


def stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def values():
    return torch.from_numpy(wl.int_uniform(N, 0, 16, seed=901)).to(DEV)


def test_scan_reports_give_up(lib):
    x = values()
    y = torch.empty_like(x)
    ws = workspace(lib.ls_scan_workspace_bytes, N, INT32, SUM)
    assert lib.scan_exclusive(x.data_ptr(), y.data_ptr(), N, INT32, SUM, None, ws.data_ptr(),
                              ws.numel(), stream()) == 0
    assert error_word(ws) & 1


def test_deterministic_scan_reports_give_up(lib):
    x = values()
    y = torch.empty_like(x)
    ws = workspace(lib.ls_scan_ex_workspace_bytes, N, INT32, SUM, DETERMINISTIC)
    assert lib.scan_ex(x.data_ptr(), y.data_ptr(), N, INT32, SUM, 1, DETERMINISTIC, None,
                       ws.data_ptr(), ws.numel(), stream()) == 0
    assert error_word(ws) & 1


def test_compaction_reports_give_up(lib):
    x = values()
    out = torch.empty_like(x)
    count = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ws = workspace(lib.ls_compact_workspace_bytes, N, INT32)
    assert lib.compact_if(x.data_ptr(), out.data_ptr(), count.data_ptr(), N, INT32, LT, 8,
                          ws.data_ptr(), ws.numel(), stream()) == 0
    assert error_word(ws) & 1
    assert 0 <= int(count.item()) <= N


def test_segmented_scan_reports_give_up(lib):
    x = values()
    y = torch.empty_like(x)
    g = np.random.default_rng(902)
    heads = torch.from_numpy((g.random(N) < 1e-5).astype(np.uint8)).to(DEV)  # most tiles hold no head
    ws = workspace(lib.ls_segmented_workspace_bytes, N, INT32, SUM)
    assert lib.segmented_scan(x.data_ptr(), y.data_ptr(), N, INT32, SUM, 0, heads.data_ptr(), None,
                              ws.data_ptr(), ws.numel(), stream()) == 0
    assert error_word(ws) & 1
