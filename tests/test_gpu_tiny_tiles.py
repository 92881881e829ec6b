"""The scans with tiny tiles: libscan_tiny.so, built by build() from the same sources
with 256-element tiles (one wave of 64 threads, one run of four elements each), so
that a few hundred elements span several tiles.

The multi-block scan of the geek-doc.cn parallel prefix scan page (section 四) splits
its 8-element example x = [3, 1, 4, 1, 5, 9, 2, 6] into two blocks of four: block
totals [9, 22], their exclusive scan [0, 9] is each block's offset, and the second
block's local exclusive result [0, 5, 14, 16] plus 9 gives [9, 14, 23, 25], the
same as one scan over all eight.  Here each block of four is the head of a tile
whose other 252 elements are 0 (the identity), and the test reads the tile totals,
the offsets and the status words the library kept in its workspace.  A random
sweep then checks every scheme against the oracle at sizes of many tiles, where
the three-phase schemes recurse over their tile totals."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "prefix_scan_stream_amd", "libscan_tiny.so")
TILE = 256
INT32, UINT32 = 0, 1
SUM, MAX = 0, 1
SINGLE, REDUCE_THEN_SCAN, SCAN_THEN_PROPAGATE, DETERMINISTIC = 0, 1, 2, 3
HEADER_BYTES, SLOT_BYTES = 256, 256
ST_AGGREGATE, ST_PREFIX = 1, 2
PAGE_X = [3, 1, 4, 1, 5, 9, 2, 6]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    szp = ctypes.POINTER(ctypes.c_size_t)
    L.ls_scan_ex_workspace_bytes.argtypes = [i64, i32, i32, i32, szp]
    L.scan_ex.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp]
    L.ls_radix_sort_workspace_bytes.argtypes = [i64, i32, i32, szp]
    L.radix_sort.argtypes = [vp, vp, vp, vp, i64, i32, vp, sz, vp]
    L.ls_workspace_init.argtypes = [vp, sz, vp]
    return L


def stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def scan(lib, x, op, exclusive, scheme):
    """Returns (out, workspace) after the call has finished."""
    n = x.numel()
    nbytes = ctypes.c_size_t(0)
    assert lib.ls_scan_ex_workspace_bytes(n, INT32, op, scheme, ctypes.byref(nbytes)) == 0
    ws = torch.zeros(max(nbytes.value, 256), dtype=torch.uint8, device=DEV)
    if scheme in (SINGLE, DETERMINISTIC):
        assert lib.ls_workspace_init(ws.data_ptr(), ws.numel(), stream()) == 0
    out = torch.full_like(x, -7)
    assert lib.scan_ex(x.data_ptr(), out.data_ptr(), n, INT32, op, int(exclusive), scheme, None,
                       ws.data_ptr(), ws.numel(), stream()) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws.cpu().numpy()


def padded(blocks):
    """Each block of values at the head of its own tile, zeros after it."""
    x = np.zeros(len(blocks) * TILE, dtype=np.int32)
    for t, b in enumerate(blocks):
        x[t * TILE:t * TILE + len(b)] = b
    return torch.from_numpy(x).to(DEV), x


@pytest.mark.parametrize("scheme", [REDUCE_THEN_SCAN, SCAN_THEN_PROPAGATE])
def test_page_two_block_decomposition_three_phase(lib, scheme):
    print(f"tiny tiles: two-block decomposition, scheme {scheme}", flush=True)
    xd, xh = padded([PAGE_X[:4], PAGE_X[4:]])
    out, ws = scan(lib, xd, SUM, True, scheme)
    totals = ws[:8].view(np.int32)
    seeds = ws[256:264].view(np.int32)  # the seeds follow the totals' 256-byte-rounded block
    assert totals.tolist() == [9, 22]
    assert seeds.tolist() == [0, 9]
    assert out[:4].tolist() == [0, 3, 4, 8]
    assert out[TILE:TILE + 4].tolist() == [9, 14, 23, 25]
    assert np.array_equal(out, oracle.scan(xh, "sum", False).y)


def test_page_two_block_decomposition_single_pass(lib):
    """The single pass keeps the same numbers in its status words: tile 0's full
    prefix 9, tile 1's total 22, and the full prefix 31 that the chasing wave
    publishes for tile 1."""
    print("tiny tiles: two-block decomposition, single pass", flush=True)
    xd, xh = padded([PAGE_X[:4], PAGE_X[4:]])
    out, ws = scan(lib, xd, SUM, True, SINGLE)
    words = ws[HEADER_BYTES:HEADER_BYTES + 2 * SLOT_BYTES].view(np.uint64).reshape(2, SLOT_BYTES // 8)

    def decode(w):
        return int(w) >> 62, int(w) & 0xFFFFFFFF

    assert decode(words[0][0]) == (ST_PREFIX, 9)      # tile 0: prefix word
    assert decode(words[0][1]) == (ST_AGGREGATE, 9)   # tile 0: total word
    assert decode(words[1][1]) == (ST_AGGREGATE, 22)  # tile 1: total word
    assert decode(words[1][0]) == (ST_PREFIX, 31)     # tile 1: chased full prefix
    assert out[TILE:TILE + 4].tolist() == [9, 14, 23, 25]
    assert np.array_equal(out, oracle.scan(xh, "sum", False).y)


def test_three_block_decomposition(lib):
    """Three blocks of four: totals [9, 22, 21], offsets [0, 9, 31]."""
    print("tiny tiles: three-block decomposition", flush=True)
    xd, xh = padded([PAGE_X[:4], PAGE_X[4:], [5, 3, 5, 8]])
    out, ws = scan(lib, xd, SUM, True, SCAN_THEN_PROPAGATE)
    assert ws[:12].view(np.int32).tolist() == [9, 22, 21]
    assert ws[256:268].view(np.int32).tolist() == [0, 9, 31]
    assert out[2 * TILE:2 * TILE + 4].tolist() == [31, 36, 39, 44]
    assert np.array_equal(out, oracle.scan(xh, "sum", False).y)


@pytest.mark.parametrize("scheme", [SINGLE, REDUCE_THEN_SCAN, SCAN_THEN_PROPAGATE, DETERMINISTIC])
@pytest.mark.parametrize("op", ["sum", "max"])
@pytest.mark.parametrize("n", [1, 255, 256, 257, 3 * 256 + 1, 65536 + 3, 256 * 256 + 256, (1 << 20) + 5])
def test_tiny_tile_sweep(lib, scheme, op, n):
    """Many tiles: at n > 65536 the three-phase schemes scan their tile totals with
    the same scheme again (more than one level)."""
    print(f"tiny tiles: scheme {scheme} {op} n={n}", flush=True)
    xh = wl.int_uniform(n, -1000, 1000, seed=n + 17 * scheme) if op == "max" else \
        wl.int_uniform(n, 0, 16, seed=n + 17 * scheme)
    xd = torch.from_numpy(xh).to(DEV)
    for exclusive in (True, False):
        out, _ = scan(lib, xd, SUM if op == "sum" else MAX, exclusive, scheme)
        assert np.array_equal(out, oracle.scan(xh, op, not exclusive).y), f"exclusive={exclusive}"


def test_sort_with_tiny_scan_tiles(lib):
    """The radix sort's digit-count scan over many tiny tiles."""
    n = (1 << 16) + 7
    print(f"tiny tiles: radix sort n={n}", flush=True)
    kh = wl.u32_bits(n, seed=5)
    kd = torch.from_numpy(kh).to(DEV)
    vd = torch.arange(n, dtype=torch.int32, device=DEV)
    ko, vo = torch.empty_like(kd), torch.empty_like(vd)
    nbytes = ctypes.c_size_t(0)
    assert lib.ls_radix_sort_workspace_bytes(n, UINT32, 1, ctypes.byref(nbytes)) == 0
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=DEV)
    assert lib.radix_sort(kd.data_ptr(), ko.data_ptr(), vd.data_ptr(), vo.data_ptr(), n, UINT32,
                          ws.data_ptr(), ws.numel(), stream()) == 0
    torch.cuda.synchronize()
    order = np.argsort(kh, kind="stable")
    assert np.array_equal(ko.cpu().numpy(), kh[order])
    assert np.array_equal(vo.cpu().numpy(), order.astype(np.int32))
