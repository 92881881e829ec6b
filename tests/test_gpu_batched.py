"""Parity of the HIP batched row scan (through the C ABI) with the CPU oracle."""
import numpy as np
import pytest

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import bits, to_dev, to_host

pytestmark = pytest.mark.gpu

COMBOS = [("int32", "sum"), ("uint32", "sum"), ("int32", "max"), ("uint32", "max"),
          ("int32", "xor"), ("float32", "sum"), ("float32", "max")]


def check_batched(x2: np.ndarray, op: str, exclusive: bool, *, offset=0, inplace=False):
    ref = oracle.batched(x2, op, inclusive=not exclusive)
    rows, cols = x2.shape
    if offset:
        flat = to_dev(np.concatenate([np.zeros(offset, x2.dtype), x2.reshape(-1)]))
        xd = flat[offset:].view(rows, cols)
    else:
        xd = to_dev(x2)
    out = ps.batched_row_scan(xd, op, exclusive, out=xd if inplace else None)
    got = to_host(out)
    if str(x2.dtype) == "float32" and op == "sum":
        ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
        assert ok, f"fp32 row sum off tolerance: ratio {worst:.3g} at flat index {k}"
    else:
        mism = np.flatnonzero(bits(got).reshape(-1) != bits(ref.y).reshape(-1))
        assert mism.size == 0, f"{mism.size} mismatches, first at flat index {mism[0]}"


@pytest.mark.parametrize("cols", [1, 2, 3, 4, 5, 16, 17, 33, 63, 64, 65, 100, 1023, 1024, 1025,
                                  2048, 5000])
@pytest.mark.parametrize("dtype,op", COMBOS)
def test_batched_matches_oracle(dtype, op, cols):
    rows = max(1, min(300, 200_000 // cols)) + 3
    x = wl.case(dtype, op, rows * cols, seed=cols).reshape(rows, cols)
    check_batched(x, op, exclusive=True)
    check_batched(x, op, exclusive=False)


@pytest.mark.parametrize("cols", [64, 1024, 60, 1000])
def test_batched_unaligned_and_inplace(cols):
    x = wl.case("int32", "sum", 77 * cols, seed=5).reshape(77, cols)
    check_batched(x, "sum", True, offset=1)
    check_batched(x, "sum", True, inplace=True)
    xf = wl.case("float32", "sum", 77 * cols, seed=6).reshape(77, cols)
    check_batched(xf, "sum", False, offset=2)


def test_batched_no_carry_between_rows():
    x = np.ones((1000, 64), np.int32)
    got = to_host(ps.batched_row_scan(to_dev(x), "sum", True))
    assert np.all(got == np.arange(64, dtype=np.int32)[None, :])


def test_rows64_workload():
    """2^20 rows x 64 float32, values U[0, 1): every element against the oracle."""
    check_batched(wl.rows64(), "sum", True)


def test_rows1024_workload():
    """2^16 rows x 1024 int32, values U{0..9}: bit-exact, every element."""
    check_batched(wl.rows1024(), "sum", True)


BLOCK_SCANS = ["wave_dpp", "hillis_steele", "hillis_steele_double", "blelloch"]


def check_variant(x2, op, exclusive, kind):
    ref = oracle.batched(x2, op, inclusive=not exclusive)
    got = to_host(ps.batched_row_scan_ex(to_dev(x2), op, exclusive, kind))
    if str(x2.dtype) == "float32" and op == "sum":
        ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
        assert ok, f"{kind}: ratio {worst:.3g} at flat index {k}"
    else:
        mism = np.flatnonzero(bits(got).reshape(-1) != bits(ref.y).reshape(-1))
        assert mism.size == 0, f"{kind}: {mism.size} mismatches, first at flat index {mism[0]}"


@pytest.mark.parametrize("cols", [1, 17, 64, 65, 255, 1023, 1024, 1025, 3000])
@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("uint32", "max"), ("int32", "max"),
                                      ("int32", "xor"), ("float32", "sum"), ("float32", "max")])
@pytest.mark.parametrize("kind", BLOCK_SCANS)
def test_block_scan_variants_match_oracle(kind, dtype, op, cols):
    rows = max(2, min(200, 100_000 // cols))
    x = wl.case(dtype, op, rows * cols, seed=cols + 3).reshape(rows, cols)
    check_variant(x, op, True, kind)
    check_variant(x, op, False, kind)


@pytest.mark.parametrize("kind", BLOCK_SCANS)
def test_block_scan_variants_rows1024_workload(kind):
    check_variant(wl.rows1024(), "sum", True, kind)

