"""Parity of the segmented scan (through the C ABI) with the CPU oracle: segments by
head flags and by CSR offsets, every operator, inclusive and exclusive.

Integer results, min/max and the affine maps must match bit for bit (the affine
maps, which do not commute, check that every combine keeps its order across heads,
runs, waves and tiles); the float32 sum must satisfy |gpu_i - ref_i| <= 1e-6 *
B_i + 1e-6 with B_i the sum of |x_j| over the segment up to i; the float32 product
the relative bound k * 2^-23 with k the elements of the segment up to i."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host, ws_error_word

pytestmark = pytest.mark.gpu

TILE = 16384
COMBOS = [("int32", "sum"), ("uint32", "sum"), ("float32", "sum"), ("int32", "max"), ("float32", "min"),
          ("uint32", "xor"), ("int32", "prod"), ("float32", "prod"), ("uint32", "and"), ("uint32", "affine")]


def make_heads(n, density, seed):
    rng = np.random.default_rng(seed)
    h = (rng.random(n) < density).astype(np.uint8)
    return h * rng.integers(1, 256, n).astype(np.uint8)   # any nonzero byte is a head


def seg_len_before(heads):
    """1-based position of each element inside its segment."""
    n = heads.size
    idx = np.arange(n)
    start = np.maximum.accumulate(np.where((heads != 0) | (idx == 0), idx, 0))
    return idx - start + 1


def check(x, op, exclusive, *, heads=None, offsets=None, xoff=0, hoff=0, inplace=False):
    dtype = str(x.dtype)
    n = x.size
    if offsets is not None:
        ref = oracle.segmented(x, op, not exclusive, offsets=offsets)
        hh = np.zeros(n, np.uint8)
        hh[offsets[:-1][offsets[:-1] < n]] = 1
    else:
        ref = oracle.segmented(x, op, not exclusive, heads=heads)
        hh = heads
    xd = to_dev(np.concatenate([np.zeros(xoff, x.dtype), x]))[xoff:] if xoff else to_dev(x)
    total = torch.empty(1, dtype=xd.dtype, device=DEV)
    kw = {}
    if offsets is not None:
        kw["offsets"] = to_dev(offsets.astype(np.int64))
    else:
        kw["heads"] = to_dev(np.concatenate([np.zeros(hoff, np.uint8), heads]))[hoff:] if hoff else to_dev(heads)
    out = ps.segmented_scan(xd, op, exclusive, out=xd if inplace else None, total=total, **kw)
    got = to_host(out)
    assert ws_error_word() == 0
    if dtype == "float32" and op == "sum":
        ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
        assert ok, f"fp32 segmented sum off tolerance: ratio {worst:.3g} at {k}"
    elif dtype == "float32" and op == "prod":
        r = np.asarray(ref.y, np.float64)
        k = seg_len_before(hh).astype(np.float64)
        bad = np.flatnonzero(np.abs(got - r) > k * 2.0 ** -23 * np.abs(r) + 1e-30)
        assert bad.size == 0, f"fp32 segmented product off bound at {bad[:3]}"
    else:
        mism = np.flatnonzero(bits(got) != bits(ref.y))
        assert mism.size == 0, f"{mism.size} mismatches, first at {mism[0]}"
    if n:
        # total: the inclusive value of element n-1, under the same rules as the elements
        incl = oracle.segmented(x, op, True, heads=hh)
        t, w = to_host(total)[0], incl.y[-1]
        if dtype == "float32" and op == "sum":
            assert abs(float(t) - float(w)) <= 1e-6 * float(incl.bound[-1]) + 1e-6
        elif dtype == "float32" and op == "prod":
            assert abs(float(t) - float(w)) <= seg_len_before(hh)[-1] * 2.0 ** -23 * abs(float(w)) + 1e-30
        else:
            assert bits(np.array([t]))[0] == bits(np.array([w], dtype=x.dtype))[0]


@pytest.mark.parametrize("n", [1, 2, 5, 64, 4097, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, 70 * TILE + 9])
@pytest.mark.parametrize("density", [0.0, 1e-5, 0.01, 0.5, 1.0])
@pytest.mark.parametrize("dtype,op", COMBOS)
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_segmented_heads_match_oracle(dtype, op, density, n, exclusive):
    x = wl.case(dtype, op, n, seed=600 + n)
    check(x, op, exclusive, heads=make_heads(n, density, n + 3))


@pytest.mark.parametrize("dtype,op", COMBOS)
def test_segmented_unaligned_and_inplace(dtype, op):
    n = 5 * TILE + 13
    x = wl.case(dtype, op, n, seed=77)
    h = make_heads(n, 0.003, 78)
    check(x, op, False, heads=h, xoff=1, hoff=3)      # 4-byte values, odd flag address: bytewise path
    check(x, op, True, heads=h, inplace=True)


@pytest.mark.parametrize("n", [1, 100, TILE + 3, 40 * TILE + 1])
@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("uint32", "affine"), ("float32", "max")])
def test_segmented_offsets_match_oracle(dtype, op, n):
    rng = np.random.default_rng(n)
    inner = np.sort(rng.integers(0, n, max(1, n // 500)))
    offsets = np.concatenate([[0], inner, inner[: len(inner) // 3], [n, n]]).astype(np.int64)
    offsets.sort()                                    # repeated offsets: empty segments
    x = wl.case(dtype, op, n, seed=n + 1)
    check(x, op, False, offsets=offsets)
    check(x, op, True, offsets=offsets)


def test_segmented_offsets_one_per_element_and_single_segment():
    n = 3 * TILE + 5
    x = wl.case("int32", "sum", n, seed=9)
    check(x, "sum", False, offsets=np.arange(n + 1, dtype=np.int64))      # every element its own segment
    check(x, "sum", True, offsets=np.array([0, n], np.int64))             # one segment: the plain scan
    got = to_host(ps.segmented_scan(to_dev(x), "sum", False, offsets=to_dev(np.array([0, n], np.int64))))
    assert np.array_equal(got, oracle.scan(x, "sum", True).y)


def test_segmented_matches_batched_rows():
    rows, cols = 300, 1000
    x = wl.case("float32", "sum", rows * cols, seed=4)
    h = np.zeros(rows * cols, np.uint8)
    h[::cols] = 1
    seg = to_host(ps.segmented_scan(to_dev(x), "sum", True, heads=to_dev(h)))
    ref = oracle.batched(x.reshape(rows, cols), "sum", inclusive=False)
    ok, worst, k = oracle.fp32_sum_within_tolerance(seg.reshape(rows, cols), ref)
    assert ok


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("float32", "max"), ("uint32", "affine")])
def test_segmented_empty_total_is_identity(dtype, op):
    tdt = {"int32": torch.int32, "uint32": torch.uint32, "float32": torch.float32}[dtype]
    x = torch.empty(0, dtype=tdt, device=DEV)
    total = torch.empty(1, dtype=tdt, device=DEV)
    ps.segmented_scan(x, op, False, heads=torch.empty(0, dtype=torch.uint8, device=DEV), total=total)
    want = {"sum": 0, "max": 0xFF800000, "affine": 0x00010000}[op]
    assert bits(to_host(total))[0] == want


def test_segmented_workload_size():
    """2^26 int32 values in segments of random length (mean 1024): every element."""
    n = 1 << 26
    x = wl.case("int32", "sum", n, seed=21)
    h = make_heads(n, 1.0 / 1024, 22)
    check(x, "sum", True, heads=h)


@pytest.mark.parametrize("density", [1e-5, 1e-3])
@pytest.mark.parametrize("by_offsets", [False, True])
def test_segmented_float_sums_repeat_bit_for_bit(density, by_offsets):
    """Carries come from chased prefixes in an order fixed by the tile index (and head
    tiles publish their own pair), so float32 sums give the same bits on every run;
    the first run is also checked against the oracle."""
    n = 300 * TILE + 7
    x = wl.fp32_scan(n)
    heads = make_heads(n, density, seed=int(density * 1e6) + 3)
    xd = to_dev(x)
    if by_offsets:
        hh = heads.copy()
        hh[0] = 1
        offs = np.concatenate([np.flatnonzero(hh), [n]]).astype(np.int64)
        od = to_dev(offs)
        run = lambda: ps.segmented_scan(xd, "sum", False, offsets=od)
        ref = oracle.segmented(x, "sum", True, offsets=offs)
    else:
        hd = to_dev(heads)
        run = lambda: ps.segmented_scan(xd, "sum", False, heads=hd)
        ref = oracle.segmented(x, "sum", True, heads=heads)
    first = to_host(run())
    ok, worst, k = oracle.fp32_sum_within_tolerance(first, ref)
    assert ok, f"ratio {worst:.3g} at {k}"
    for _ in range(3):
        assert np.array_equal(bits(to_host(run())), bits(first)), "segmented sum changed between runs"
    assert ws_error_word() == 0
