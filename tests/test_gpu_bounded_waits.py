"""Bounded waits end with a correct result or a report, never a hang.

Every wait of one tile on another is bounded in time.  What happens when the time
runs out depends on how tiles reach blocks:
  - block-index tiles (the plain single-pass scan and the compaction) compute what
    they waited for themselves, from the input: the scan replays the chasing
    wave's arithmetic (the same bits), the compaction recounts the missing tiles.
    The result stays exact and nothing is reported;
  - ticket tiles (the fixed-order scan, the segmented scan) give up, set bit 0 of
    the workspace error word, and ls_workspace_check reports LS_ERR_INCOMPLETE; the
    call's outputs are then unspecified.  ls_workspace_init clears the report.
prefix_scan_stream_amd/libscan_spin1.so (built by build() from the same sources)
runs out of time at the first empty poll of every wait, so in a multi-tile call
these paths are certain to run.

Only entry points whose stores stay inside their buffers whatever a tile's offset
are called on the ticket paths: scan tiles write through their own byte range.
The radix sort is left out: its scatter addresses come from its scan."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "prefix_scan_stream_amd", "libscan_spin1.so")
INT32, UINT32, F32 = 0, 1, 2
SUM, MAX, AFFINE = 0, 1, 7
LT, DETERMINISTIC, INCOMPLETE = 0, 3, 5
N = 1 << 25            # hundreds of tiles: the ticket paths
N_FALLBACK = (1 << 22) + 12345  # 158 scan tiles, 257 compaction tiles: the forced fallbacks


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
    L.scan_inclusive.argtypes = [vp, vp, i64, i32, i32, vp, vp, sz, vp]
    L.scan_ex.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp]
    L.compact_if.argtypes = [vp, vp, vp, i64, i32, i32, u32, vp, sz, vp]
    L.segmented_scan.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp, sz, vp]
    L.ls_workspace_init.argtypes = [vp, sz, vp]
    L.ls_workspace_check.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    return L


_LIB = None


@pytest.fixture(autouse=True)
def _bind(lib):
    global _LIB
    _LIB = lib
    yield


def stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def workspace(query, *args):
    nbytes = ctypes.c_size_t(0)
    assert query(*args, ctypes.byref(nbytes)) == 0
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=DEV)
    assert _LIB.ls_workspace_init(ws.data_ptr(), ws.numel(), stream()) == 0
    return ws


def error_word(ws):
    """Through the C ABI; the call waits for the stream, so every kernel has ended."""
    flags = ctypes.c_uint32(0)
    st = _LIB.ls_workspace_check(ws.data_ptr(), ctypes.byref(flags), stream())
    assert st == (INCOMPLETE if flags.value else 0)
    return flags.value


def values(n=N, seed=901):
    return torch.from_numpy(wl.int_uniform(n, 0, 16, seed=seed)).to(DEV)


# ------------------------------------------------ block-index tiles: exact fallbacks

@pytest.mark.parametrize("dtype,op,inclusive", [("int32", "sum", False), ("float32", "sum", True),
                                                ("int32", "max", True), ("float32", "max", False),
                                                ("uint32", "affine", True)])
def test_scan_fallback_replays_the_same_bits(lib, dtype, op, inclusive):
    """Every tile replays its prefix instead of waiting: the result is the oracle's
    (integers, max, affine maps: the replay combines in element order) and the same
    bits as the normal library's (float sums)."""
    print(f"forced-fallback scan {dtype} {op} inclusive={inclusive} n={N_FALLBACK}", flush=True)
    xh = wl.case(dtype, op, N_FALLBACK, seed=930)
    x = torch.from_numpy(xh).to(DEV)
    y = torch.empty_like(x)
    t = {"int32": INT32, "uint32": UINT32, "float32": F32}[dtype]
    o = {"sum": SUM, "max": MAX, "affine": AFFINE}[op]
    ws = workspace(lib.ls_scan_workspace_bytes, N_FALLBACK, t, o)
    for rep in range(2):  # the second call runs under the next epoch of the same workspace
        y.fill_(7)
        fn = lib.scan_inclusive if inclusive else lib.scan_exclusive
        assert fn(x.data_ptr(), y.data_ptr(), N_FALLBACK, t, o, None, ws.data_ptr(), ws.numel(), stream()) == 0
        assert error_word(ws) == 0
        got = y.cpu().numpy()
        want = (ps.scan_inclusive if inclusive else ps.scan_exclusive)(x, op).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"call {rep}"
        if dtype != "float32":
            assert np.array_equal(got, oracle.scan(xh, op, inclusive).y)


@pytest.mark.parametrize("sel", [0.01, 0.5])
def test_compaction_fallback_recounts_exactly(lib, sel):
    print(f"forced-fallback compaction sel={sel} n={N_FALLBACK}", flush=True)
    xh = wl.compact_input(N_FALLBACK)
    thr = wl.threshold_for(sel)
    x = torch.from_numpy(xh).to(DEV)
    out = torch.full_like(x, -1)
    count = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ws = workspace(lib.ls_compact_workspace_bytes, N_FALLBACK, INT32)
    assert lib.compact_if(x.data_ptr(), out.data_ptr(), count.data_ptr(), N_FALLBACK, INT32, LT, thr,
                          ws.data_ptr(), ws.numel(), stream()) == 0
    assert error_word(ws) == 0
    want, wc = oracle.compact(xh, "lt", thr)
    c = int(count.item())
    assert c == wc
    assert np.array_equal(out.cpu().numpy()[:c], want)


# ------------------------------------------------ ticket tiles: reported give-ups

def float_values():
    return torch.from_numpy(wl.fp32_scan(N)).to(DEV)


def fixed_order_scan(lib, x, y, ws):
    """float32 sum with the fixed-order scheme: its own kernel, on tickets (for the
    other operators that scheme is the plain single pass)."""
    assert lib.scan_ex(x.data_ptr(), y.data_ptr(), N, F32, SUM, 0, DETERMINISTIC, None,
                       ws.data_ptr(), ws.numel(), stream()) == 0


def test_init_clears_the_report(lib):
    x = float_values()
    y = torch.empty_like(x)
    ws = workspace(lib.ls_scan_ex_workspace_bytes, N, F32, SUM, DETERMINISTIC)
    assert error_word(ws) == 0
    fixed_order_scan(lib, x, y, ws)
    assert error_word(ws) & 1
    assert lib.ls_workspace_init(ws.data_ptr(), ws.numel(), stream()) == 0
    assert error_word(ws) == 0


def test_deterministic_scan_reports_give_up(lib):
    x = float_values()
    y = torch.empty_like(x)
    ws = workspace(lib.ls_scan_ex_workspace_bytes, N, F32, SUM, DETERMINISTIC)
    fixed_order_scan(lib, x, y, ws)
    assert error_word(ws) & 1


def test_segmented_scan_reports_give_up(lib):
    x = values()
    y = torch.empty_like(x)
    g = np.random.default_rng(902)
    heads = torch.from_numpy((g.random(N) < 1e-5).astype(np.uint8)).to(DEV)  # most tiles hold no head
    ws = workspace(lib.ls_segmented_workspace_bytes, N, INT32, SUM)
    assert lib.segmented_scan(x.data_ptr(), y.data_ptr(), N, INT32, SUM, 0, heads.data_ptr(), None,
                              ws.data_ptr(), ws.numel(), stream()) == 0
    assert error_word(ws) & 1


def test_checked_binding_raises_on_a_flagged_workspace():
    """In checked mode the binding reads the error word after each call: a clean
    call returns normally; a workspace whose error bit is set (as a give-up sets it)
    makes the call raise LS_ERR_INCOMPLETE and is initialised again."""
    x = values()
    want = torch.cumsum(x.to(torch.int64), 0).to(torch.int32) - x
    ps.set_checked(True)
    try:
        assert torch.equal(ps.scan_exclusive(x, "sum"), want)
        ws = ps.workspace_for(DEV, torch.cuda.current_stream(DEV), 0)
        ws[8] = 1  # bit 0 of the header's error word
        with pytest.raises(ps.LibscanError) as err:
            ps.scan_exclusive(x, "sum")
        assert err.value.status == ps.LS_ERR_INCOMPLETE
        assert ps.workspace_error_flags(DEV) == 0
        assert torch.equal(ps.scan_exclusive(x, "sum"), want)
    finally:
        ps.set_checked(False)
