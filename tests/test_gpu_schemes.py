"""Parity of the three device-wide schemes (single pass, reduce-then-scan,
scan-then-propagate) through scan_ex, against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host, ws_error_word

pytestmark = pytest.mark.gpu

TILE = 16384  # the three-phase schemes' tile; the sizes span tiles, ragged tails and many tiles
SP_TILE = 32768  # the deterministic single pass's tile (groups of 64 such tiles)
SCHEMES = ["single_pass", "reduce_then_scan", "scan_then_propagate", "deterministic"]
COMBOS = [("int32", "sum"), ("uint32", "xor"), ("int32", "max"), ("uint32", "max"),
          ("float32", "sum"), ("float32", "max")]


def check(x, op, inclusive, scheme, *, offset=0, inplace=False):
    ref = oracle.scan(x, op, inclusive)
    if offset:
        xd = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))[offset:]
    else:
        xd = to_dev(x)
    total = torch.empty(1, dtype=xd.dtype, device=DEV)
    out = ps.scan_ex(xd, op, inclusive, scheme, out=xd if inplace else None, total=total)
    got, tot = to_host(out), to_host(total)
    if str(x.dtype) == "float32" and op == "sum":
        ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
        assert ok, f"{scheme}: ratio {worst:.3g} at {k}"
    else:
        mism = np.flatnonzero(bits(got) != bits(ref.y))
        assert mism.size == 0, f"{scheme}: {mism.size} mismatches, first at {mism[0]}"
        assert bits(tot)[0] == bits(np.array([ref.total], x.dtype))[0]


@pytest.mark.parametrize("n", [1, 2, 63, 4097, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, 300_003,
                               SP_TILE - 1, SP_TILE + 1, 77 * TILE + 13])
@pytest.mark.parametrize("dtype,op", COMBOS)
@pytest.mark.parametrize("scheme", SCHEMES)
@pytest.mark.parametrize("inclusive", [True, False], ids=["incl", "excl"])
def test_scheme_matches_oracle(inclusive, scheme, dtype, op, n):
    check(wl.case(dtype, op, n, seed=n + 5), op, inclusive, scheme)


@pytest.mark.parametrize("scheme", SCHEMES)
def test_scheme_unaligned_inplace(scheme):
    x = wl.case("int32", "sum", 5 * TILE + 3, seed=9)
    check(x, "sum", True, scheme, offset=1)
    check(x, "sum", False, scheme, inplace=True)
    xf = wl.case("float32", "sum", 5 * TILE + 3, seed=10)
    check(xf, "sum", False, scheme, offset=3)


@pytest.mark.parametrize("scheme", ["reduce_then_scan", "scan_then_propagate"])
def test_three_phase_recursive_totals(scheme):
    """More than TILE tiles: the tile totals are themselves scanned in three phases."""
    n = TILE * TILE + 3 * TILE + 5
    x = wl.int_uniform(n, 0, 16, seed=31)
    check(x, "sum", False, scheme)


@pytest.mark.parametrize("scheme", SCHEMES)
def test_scheme_big_scan_workload(scheme):
    check(wl.big_scan(), "sum", False, scheme)


GROUP = 64  # single-pass tiles per group of the deterministic scheme


@pytest.mark.parametrize("op", ["sum", "prod"])
@pytest.mark.parametrize("n", [SP_TILE * GROUP - 1, SP_TILE * GROUP + 1, 3 * SP_TILE * GROUP + 17,
                               1 << 26])
def test_deterministic_scheme_is_bitwise_reproducible(op, n):
    """Float sums and products under the fixed-order single pass: within the
    tolerance of the oracle, and the same bits on every one of several runs."""
    x = wl.case("float32", op, n, seed=n + 11)
    xd = to_dev(x)
    first = None
    for _ in range(4):
        got = to_host(ps.scan_ex(xd, op, True, "deterministic"))
        if first is None:
            first = got.copy()
            ref = oracle.scan(x, op, True)
            if op == "sum":
                ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
                assert ok, f"ratio {worst:.3g} at {k}"
            else:
                r = ref.y
                k = np.arange(1, n + 1, dtype=np.float64)
                assert np.all(np.abs(got - r) <= k * 2.0 ** -23 * np.abs(r) + 1e-30)
        else:
            assert np.array_equal(bits(got), bits(first)), "deterministic scan changed between runs"


CHASED_TILE = 28672  # the plain single pass's tile; its prefixes come in groups of 64 tiles


@pytest.mark.parametrize("op", ["sum", "prod"])
@pytest.mark.parametrize("n", [64 * CHASED_TILE - 1, 64 * CHASED_TILE + 1, 3 * 64 * CHASED_TILE + 7,
                               700 * CHASED_TILE + 5])
def test_default_single_pass_is_bitwise_reproducible(op, n):
    """The plain single pass publishes tile prefixes in groups of 64 tiles aligned to
    tile 0, each prefix a fixed function of the tile totals: float sums and products
    give the same bits on every run, and stay within the oracle's tolerance."""
    x = wl.case("float32", op, n, seed=n + 17)
    xd = to_dev(x)
    first = None
    for _ in range(4):
        got = to_host(ps.scan_inclusive(xd, op))
        if first is None:
            first = got.copy()
            ref = oracle.scan(x, op, True)
            if op == "sum":
                ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
                assert ok, f"ratio {worst:.3g} at {k}"
            else:
                r = ref.y
                k = np.arange(1, n + 1, dtype=np.float64)
                assert np.all(np.abs(got - r) <= k * 2.0 ** -23 * np.abs(r) + 1e-30)
        else:
            assert np.array_equal(bits(got), bits(first)), "single-pass scan changed between runs"
        assert ws_error_word() == 0


@pytest.mark.parametrize("n", [GROUP * SP_TILE - 1, GROUP * SP_TILE, GROUP * SP_TILE + 1,
                               2 * GROUP * SP_TILE + SP_TILE + 3, 300 * TILE + 5])
def test_deterministic_scheme_keeps_order(n):
    """Affine maps take the fixed-order kernel too: any combine out of order (the
    group prefix on the wrong side, a total of the wrong tile) changes the bits."""
    x = wl.case("uint32", "affine", n, seed=n + 13)
    check(x, "affine", True, "deterministic")
    check(x, "affine", False, "deterministic")
