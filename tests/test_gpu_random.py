"""Randomized parity sweep (through the C ABI) against the CPU oracle.

Each case draws its entry point's parameters from one seed: the size (log-uniform
from 0 to about 5 million elements, so tile and group boundaries fall anywhere),
the dtype and operator, inclusive or exclusive, the device-wide scheme, the
comparison and selectivity of a compaction, the density of segment heads, and
whether a sort carries values.  The parity bar is the one of the dedicated tests:
integers, min / max, affine maps, compaction and sorting bit for bit; float32 sums
within 1e-6 * sum|x| + 1e-6 of the fp64 oracle; float32 products within
k * 2^-23 relative.  A failing case names its seed, so it can be rerun alone."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host, ws_error_word

pytestmark = pytest.mark.gpu

SCAN_COMBOS = [("int32", op) for op in ("sum", "max", "min", "xor", "and", "or", "prod")] + \
              [("uint32", op) for op in ("sum", "max", "min", "xor", "and", "or", "prod", "affine")] + \
              [("float32", op) for op in ("sum", "max", "min", "prod")]
SCHEMES = ["single_pass", "single_pass", "deterministic", "reduce_then_scan", "scan_then_propagate"]
CMPS = ["lt", "le", "gt", "ge", "eq", "ne"]


def draw_n(g, top=6.7):
    return int(10 ** g.uniform(0.0, top)) - 1


def assert_scan(got, ref, dtype, op, seed, seg_pos=None):
    if dtype == "float32" and op == "sum":
        ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
        assert ok, f"seed {seed}: fp32 sum off by {worst:.3g} of the bound at {k}"
    elif dtype == "float32" and op == "prod":
        g = np.asarray(got, np.float64)
        r = np.asarray(ref.y, np.float64)
        k = (np.arange(r.size) + 1.0) if seg_pos is None else seg_pos.astype(np.float64)
        bad = np.flatnonzero(np.abs(g - r) > k * 2.0 ** -23 * np.abs(r) + 1e-30)
        assert bad.size == 0, f"seed {seed}: fp32 product off bound at {bad[:3]}"
    else:
        mism = np.flatnonzero(bits(got) != bits(ref.y))
        assert mism.size == 0, f"seed {seed}: {mism.size} mismatches, first at {mism[:3]}"


@pytest.mark.parametrize("seed", range(300))
def test_random_scan(seed):
    g = np.random.default_rng(10_000 + seed)
    dtype, op = SCAN_COMBOS[g.integers(len(SCAN_COMBOS))]
    n = draw_n(g)
    inclusive = bool(g.integers(2))
    scheme = SCHEMES[g.integers(len(SCHEMES))]
    x = wl.case(dtype, op, n, seed=20_000 + seed)
    ref = oracle.scan(x, op, inclusive)
    out = ps.scan_ex(to_dev(x), op, inclusive, scheme)
    # the error word belongs to calls that ran a look-back kernel (n > 0; three-phase
    # schemes keep tile totals in the same workspace instead)
    if scheme in ("single_pass", "deterministic") and n:
        assert ws_error_word() == 0, f"seed {seed}: look-back error word set"
    assert_scan(to_host(out), ref, dtype, op, seed)


@pytest.mark.parametrize("seed", range(100))
def test_random_compaction(seed):
    g = np.random.default_rng(30_000 + seed)
    dtype = ["int32", "uint32", "float32"][g.integers(3)]
    cmp = CMPS[g.integers(len(CMPS))]
    n = draw_n(g)
    if dtype == "float32":
        x = g.integers(-50, 50, n).astype(np.float32) * np.float32(0.5)
        x[g.random(n) < 0.05] = -0.0
    elif dtype == "int32":
        x = g.integers(-1000, 1000, n).astype(np.int32)
    else:
        x = g.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    thr = x[g.integers(n)] if n else x.dtype.type(0)   # an existing value: "eq" and "ne" matter
    want, wc = oracle.compact(x, cmp, thr)
    out = to_dev(np.full(n, 0xDEADBEEF, np.uint32).view(x.dtype))
    cnt = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ps.compact_if(to_dev(x), cmp, thr, out=out, count=cnt)
    got = to_host(out)
    c = int(to_host(cnt)[0])
    assert c == wc, f"seed {seed}: count {c} != {wc}"
    assert np.array_equal(bits(got[:c]), bits(want)), f"seed {seed}: kept elements differ"
    assert np.all(bits(got[c:]) == 0xDEADBEEF), f"seed {seed}: wrote past the count"
    if n:
        assert ws_error_word() == 0


@pytest.mark.parametrize("seed", range(100))
def test_random_segmented(seed):
    g = np.random.default_rng(40_000 + seed)
    combos = [("int32", "sum"), ("uint32", "max"), ("float32", "sum"), ("float32", "min"),
              ("uint32", "affine"), ("int32", "prod")]
    dtype, op = combos[g.integers(len(combos))]
    n = draw_n(g, 6.5)
    exclusive = bool(g.integers(2))
    density = 10 ** g.uniform(-5.0, -0.3)
    x = wl.case(dtype, op, n, seed=50_000 + seed)
    heads = ((g.random(n) < density) * g.integers(1, 256, n)).astype(np.uint8)
    by_offsets = bool(g.integers(2))
    if by_offsets:
        hh = heads.copy()
        if n:
            hh[0] = 1
        offs = np.concatenate([np.flatnonzero(hh), [n]]).astype(np.int64)
        ref = oracle.segmented(x, op, not exclusive, offsets=offs)
        out = ps.segmented_scan(to_dev(x), op, exclusive, offsets=to_dev(offs))
    else:
        hh = heads
        ref = oracle.segmented(x, op, not exclusive, heads=heads)
        out = ps.segmented_scan(to_dev(x), op, exclusive, heads=to_dev(heads))
    idx = np.arange(n)
    start = np.maximum.accumulate(np.where((hh != 0) | (idx == 0), idx, 0)) if n else idx
    assert_scan(to_host(out), ref, dtype, op, seed, seg_pos=idx - start + 1)
    if n:
        assert ws_error_word() == 0


@pytest.mark.parametrize("seed", range(40))
def test_random_sort(seed):
    g = np.random.default_rng(60_000 + seed)
    dtype = ["int32", "uint32", "float32"][g.integers(3)]
    n = draw_n(g, 6.3)
    k = wl.u32_bits(n, seed=70_000 + seed)
    if g.integers(2) and n:
        k = k[g.integers(0, max(1, n // 50), n)]          # many equal keys
    keys = k.view(np.int32) if dtype == "int32" else (k.view(np.float32) if dtype == "float32" else k)
    with_values = bool(g.integers(2))
    vals = np.arange(n, dtype=np.uint32) if with_values else None
    wk, wv = oracle.sort(keys, vals)
    gk, gv = ps.radix_sort(to_dev(keys), to_dev(vals) if with_values else None)
    assert np.array_equal(bits(to_host(gk)), bits(wk)), f"seed {seed}: keys differ"
    if with_values:
        assert np.array_equal(to_host(gv), wv), f"seed {seed}: values differ (stability)"
