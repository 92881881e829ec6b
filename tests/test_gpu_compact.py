"""Parity of the fused HIP compaction (through the C ABI) with the CPU oracle:
bit-exact kept elements, in input order, exact count, and no write past the count."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host, ws_error_word

pytestmark = pytest.mark.gpu

TILE = 16384  # the library's compaction tile; sizes below also cover half and quarter tiles
SENTINEL = 0xDEADBEEF


def check_compact(x: np.ndarray, cmp: str, thr, *, offset=0):
    want, wc = oracle.compact(x, cmp, thr)
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
    else:
        xd = to_dev(x)
    out = to_dev(np.full(x.size, SENTINEL, np.uint32).view(x.dtype))
    count = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.compact_if(xd, cmp, thr, out=out, count=count)
    got = to_host(out)
    c = int(to_host(count)[0])
    assert ws_error_word() == 0
    assert c == wc
    assert np.array_equal(bits(got[:c]), bits(want))
    assert np.all(bits(got[c:]) == SENTINEL), "wrote beyond the count"


@pytest.mark.parametrize("n", [1, 2, 17, 64, 4095, 4096, 4097, 8191, TILE - 1, TILE, TILE + 1, 2 * TILE - 1,
                               2 * TILE + 1, 3 * TILE + 5, 70 * TILE + 9, 200_003, 300 * TILE + 11,
                               1100 * TILE + 7])
@pytest.mark.parametrize("dtype", ["int32", "uint32", "float32"])
@pytest.mark.parametrize("cmp", ["lt", "le", "gt", "ge", "eq", "ne"])
def test_compact_matches_oracle(dtype, cmp, n):
    rng = np.random.default_rng(n)
    if dtype == "float32":
        x = rng.integers(-4, 5, n).astype(np.float32)
        x[::7] = -0.0
        thr = np.float32(0.0)
    elif dtype == "int32":
        x = rng.integers(-4, 5, n).astype(np.int32)
        thr = np.int32(1)
    else:
        x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        x[::3] = 0x80000000
        thr = np.uint32(0x80000000)
    check_compact(x, cmp, thr)


@pytest.mark.parametrize("sel", [0.0, 0.01, 0.5, 0.99, 1.0])
def test_compact_selectivities(sel):
    x = wl.compact_input(1 << 20)
    thr = (1 << 31) - 1 if sel == 1.0 else wl.threshold_for(sel)
    cmp = "le" if sel == 1.0 else "lt"
    check_compact(x, cmp, np.int32(thr))


def test_compact_mixed_density_tiles():
    """One call over regions that keep 1, 24, 26, 60, 99, 0 and 100 % of their elements,
    each one to three tiles long and ragged, in turn: tiles that keep under a quarter of
    their elements look back 32 status words per poll, the others 8, so both kinds of
    look-back meet in one chain."""
    rng = np.random.default_rng(2024)
    fracs = [0.01, 0.24, 0.26, 0.6, 0.99, 0.0, 1.0]
    parts = []
    for i in range(70):
        m = int(rng.integers(1, 4)) * TILE + int(rng.integers(0, 100))
        keep = rng.random(m) < fracs[i % len(fracs)]
        parts.append(np.where(keep, rng.integers(0, 1000, m), rng.integers(1000, 1 << 31, m)).astype(np.int32))
    check_compact(np.concatenate(parts), "lt", np.int32(1000))


def test_compact_unaligned_input():
    x = wl.compact_input(9 * TILE + 3)
    check_compact(x, "lt", np.int32(wl.threshold_for(0.5)), offset=1)


def test_compact_nan_and_signed_zero():
    x = np.array([np.nan, 0.0, -0.0, 1.0, np.nan, -1.0] * 1000, np.float32)
    for cmp in ("lt", "le", "gt", "ge", "eq", "ne"):
        check_compact(x, cmp, np.float32(0.0))


def test_compact_empty():
    x = torch.empty(0, dtype=torch.int32, device=DEV)
    count = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.compact_if(x, "lt", 3, count=count)
    assert int(to_host(count)[0]) == 0


def test_compact_worked_example():
    out, count = ps.compact_if(to_dev(wl.WORKED_EXAMPLE), "gt", 2)
    c = int(to_host(count)[0])
    assert c == 5 and to_host(out)[:c].tolist() == [3, 4, 5, 9, 6]


@pytest.mark.parametrize("sel", wl.SELECTIVITIES)
def test_compact_workload_full_compare(sel):
    """int32, N = 2^27, values U[0, 2^31), x < round(sel * 2^31): full compare."""
    x = wl.compact_input()
    check_compact(x, "lt", np.int32(wl.threshold_for(sel)))
