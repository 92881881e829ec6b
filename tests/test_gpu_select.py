"""Parity of compaction by a flag array and of index selection (through the C ABI)
with the CPU oracle: bit-exact outputs and counts, nothing written past the count."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host

pytestmark = pytest.mark.gpu

TILE = 16384  # the library's compaction tile
SENTINEL = 0xDEADBEEF
SIZES = [1, 2, 3, 17, 4095, 4096, 4097, TILE - 1, TILE, TILE + 1, 2 * TILE - 1, 2 * TILE + 1, 3 * TILE + 5, 300_007]


def flags_for(n, seed, p):
    rng = np.random.default_rng(seed)
    return ((rng.random(n) < p) * rng.integers(1, 256, n)).astype(np.uint8)


def check_out(got_t, count_t, want, wc):
    got = to_host(got_t)
    c = int(to_host(count_t)[0])
    assert c == wc
    assert np.array_equal(bits(got[:c]), bits(want))
    assert np.all(bits(got[c:]) == SENTINEL), "wrote beyond the count"


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("p", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("flag_offset", [0, 1], ids=["flags4", "flags_unaligned"])
def test_compact_flags(n, p, flag_offset):
    x = wl.u32_bits(n, seed=n).view(np.float32)      # payload bits of any kind
    f = flags_for(n, n + 1, p)
    want, wc = oracle.compact_flags(x, f)
    fd = to_dev(np.concatenate([np.zeros(flag_offset, np.uint8), f]))[flag_offset:]
    out = to_dev(np.full(n, SENTINEL, np.uint32).view(np.float32))
    cnt = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.compact_flags(to_dev(x), fd, out=out, count=cnt)
    check_out(out, cnt, want, wc)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("p", [0.0, 0.3, 1.0])
def test_select_indices_flags(n, p):
    f = flags_for(n, n + 2, p)
    want, wc = oracle.indices(flags=f)
    out = to_dev(np.full(n, SENTINEL, np.uint32).view(np.int32))
    cnt = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.select_indices_flags(to_dev(f), out=out, count=cnt)
    check_out(out, cnt, want.view(np.int32), wc)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,cmp,thr", [("int32", "lt", 0), ("uint32", "ge", 0x80000000),
                                           ("float32", "ne", 0.0), ("int32", "eq", 3)])
def test_select_indices_if(n, dtype, cmp, thr):
    rng = np.random.default_rng(n + 7)
    if dtype == "float32":
        x = rng.integers(-2, 3, n).astype(np.float32)
        x[::9] = np.nan
    elif dtype == "int32":
        x = rng.integers(-5, 6, n).astype(np.int32)
    else:
        x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    want, wc = oracle.indices(x=x, cmp=cmp, threshold=thr)
    out = to_dev(np.full(n, SENTINEL, np.uint32).view(np.int32))
    cnt = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.select_indices_if(to_dev(x), cmp, thr, out=out, count=cnt)
    check_out(out, cnt, want.view(np.int32), wc)


def test_worked_example_flags_and_indices():
    x = to_dev(wl.WORKED_EXAMPLE)
    f = to_dev(np.array([1, 0, 1, 0, 1, 1, 0, 1], np.uint8))
    out, c = ps.compact_flags(x, f)
    assert to_host(out)[:int(to_host(c)[0])].tolist() == [3, 4, 5, 9, 6]
    idx, c = ps.select_indices_flags(f)
    assert to_host(idx)[:int(to_host(c)[0])].tolist() == [0, 2, 4, 5, 7]
    idx, c = ps.select_indices_if(x, "gt", 2)
    assert to_host(idx)[:int(to_host(c)[0])].tolist() == [0, 2, 4, 5, 7]


def test_flags_workload_size():
    n = 1 << 27
    f = flags_for(n, 5, 0.5)
    x = wl.compact_input()
    want, wc = oracle.compact_flags(x, f)
    out, cnt = ps.compact_flags(to_dev(x), to_dev(f))
    assert int(to_host(cnt)[0]) == wc
    assert np.array_equal(to_host(out)[:wc], want)


MANY = 700 * TILE + 13  # more tiles than one wave of resident blocks: blocks loop over tiles


@pytest.mark.parametrize("p", [0.02, 0.5, 0.98])
def test_many_tiles_per_block(p):
    """Flag compaction and both index selections where every block handles several
    tiles in turn (its next tile counted while the current one is copied out)."""
    n = MANY
    f = flags_for(n, 91, p)
    x = wl.u32_bits(n, seed=92).view(np.float32)
    want, wc = oracle.compact_flags(x, f)
    out = to_dev(np.full(n, SENTINEL, np.uint32).view(np.float32))
    cnt = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.compact_flags(to_dev(x), to_dev(f), out=out, count=cnt)
    check_out(out, cnt, want, wc)

    want, wc = oracle.indices(flags=f)
    out = to_dev(np.full(n, SENTINEL, np.uint32).view(np.int32))
    ps.select_indices_flags(to_dev(f), out=out, count=cnt)
    check_out(out, cnt, want.view(np.int32), wc)

    xi = wl.u32_bits(n, seed=93).view(np.int32)
    thr = int(np.quantile(xi, p))
    want, wc = oracle.indices(x=xi, cmp="lt", threshold=thr)
    out = to_dev(np.full(n, SENTINEL, np.uint32).view(np.int32))
    ps.select_indices_if(to_dev(xi), "lt", thr, out=out, count=cnt)
    check_out(out, cnt, want.view(np.int32), wc)
