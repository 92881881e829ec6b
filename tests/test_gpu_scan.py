"""Parity of the HIP device-wide scan (through the C ABI) with the CPU oracle.

Integer scans and every max scan must match bit for bit; the float32 sum must
satisfy |gpu_i - ref_i| <= 1e-6 * sum_{j<=i}|x_j| + 1e-6 against the oracle's
float64 accumulation.  Sizes span one tile (4096 elements), several tiles with a
ragged tail, look-back windows longer than 64 tiles, and the full workloads."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host, ws_error_word

pytestmark = pytest.mark.gpu

TILE = 8192      # a quarter of the deterministic single pass's tile (32768)
SP_TILE = 28672  # the single pass's tile; the chasing wave reads 64 tiles per poll
SIZES = [1, 2, 3, 63, 64, 65, 255, 256, 1023, 4095, 4096, 4097, TILE - 1, TILE, TILE + 1,
         2 * TILE - 1, 2 * TILE + 1, 4 * TILE - 1, 4 * TILE, 4 * TILE + 1,
         3 * TILE + 7, 64 * TILE, 257 * TILE + 5, 300_003, 600 * TILE + 3,
         SP_TILE - 1, SP_TILE, SP_TILE + 1, 2 * SP_TILE + 1, 65 * SP_TILE, 66 * SP_TILE + 1,
         700 * SP_TILE + 5]
COMBOS = [("int32", "sum"), ("uint32", "sum"), ("int32", "max"), ("uint32", "max"),
          ("int32", "xor"), ("uint32", "xor"), ("float32", "sum"), ("float32", "max")]


def check_scan(x: np.ndarray, op: str, inclusive: bool, *, offset=0, inplace=False):
    dtype = str(x.dtype)
    ref = oracle.scan(x, op, inclusive)
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
    else:
        xd = to_dev(x)
    total = torch.empty(1, dtype=xd.dtype, device=DEV)
    fn = ps.scan_inclusive if inclusive else ps.scan_exclusive
    out = fn(xd, op, out=xd if inplace else None, total=total)
    got = to_host(out)
    tot = to_host(total)
    assert ws_error_word() == 0
    if dtype == "float32" and op == "sum":
        ok, worst, k = oracle.fp32_sum_within_tolerance(got, ref)
        assert ok, f"fp32 sum off tolerance: ratio {worst:.3g} at {k}"
        if x.size:
            tref = oracle.ScanResult(np.array([ref.total]), None, ref.bound[-1:])
            assert oracle.fp32_sum_within_tolerance(tot, tref)[0]
    else:
        mism = np.flatnonzero(bits(got) != bits(ref.y))
        assert mism.size == 0, f"{mism.size} mismatches, first at {mism[0]}"
        assert bits(tot)[0] == bits(np.array([ref.total], dtype=x.dtype))[0]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,op", COMBOS)
@pytest.mark.parametrize("inclusive", [True, False], ids=["incl", "excl"])
def test_scan_matches_oracle(dtype, op, inclusive, n):
    x = wl.case(dtype, op, n, seed=1000 + n)
    check_scan(x, op, inclusive)


@pytest.mark.parametrize("dtype,op", COMBOS)
def test_scan_unaligned_and_inplace(dtype, op):
    x = wl.case(dtype, op, 5 * TILE + 13, seed=77)
    check_scan(x, op, True, offset=1)      # 4-byte aligned only: element path
    check_scan(x, op, False, offset=3)
    check_scan(x, op, True, inplace=True)
    check_scan(x, op, False, inplace=True)


@pytest.mark.parametrize("dtype,op", COMBOS)
def test_scan_empty_writes_identity_total(dtype, op):
    tdt = {"int32": torch.int32, "uint32": torch.uint32, "float32": torch.float32}[dtype]
    x = torch.empty(0, dtype=tdt, device=DEV)
    total = torch.full((1,), 7, dtype=tdt, device=DEV) if dtype != "uint32" else \
        torch.from_numpy(np.array([7], np.uint32)).to(DEV)
    ps.scan_exclusive(x, op, total=total)
    got = bits(to_host(total))[0]
    want = {"sum": 0, "xor": 0}.get(op)
    if op == "max":
        want = {"int32": 0x80000000, "uint32": 0, "float32": 0xFF800000}[dtype]
    assert got == want


def test_float_xor_unsupported():
    x = torch.zeros(16, dtype=torch.float32, device=DEV)
    with pytest.raises(ps.LibscanError) as e:
        ps.scan_inclusive(x, "xor")
    assert e.value.status == ps.LS_ERR_UNSUPPORTED


def test_worked_example_on_gpu():
    x = wl.WORKED_EXAMPLE
    assert to_host(ps.scan_inclusive(to_dev(x))).tolist() == [3, 4, 8, 9, 14, 23, 25, 31]
    assert to_host(ps.scan_exclusive(to_dev(x))).tolist() == [0, 3, 4, 8, 9, 14, 23, 25]


def test_exact_float_special_case():
    """Integer-valued float32 data with all partial sums below 2^24 adds exactly in any
    order, so the GPU must match the oracle bit for bit there."""
    rng = np.random.default_rng(4)
    x = rng.integers(-8, 9, 300 * TILE + 3).astype(np.float32)
    ref = oracle.scan(x, "sum", True)
    assert np.max(np.abs(ref.y)) < 2 ** 24
    got = to_host(ps.scan_inclusive(to_dev(x)))
    assert np.array_equal(got.astype(np.float64), ref.y)


def test_repeated_calls_are_stable():
    """The same scan many times in a row: a race in the look-back would show up as a
    rare mismatch."""
    x = wl.small_scan()
    ref = oracle.scan(x, "sum", False).y
    xd = to_dev(x)
    out = torch.empty_like(xd)
    for _ in range(100):
        ps.scan_exclusive(xd, out=out)
        assert np.array_equal(to_host(out), ref)
    assert ws_error_word() == 0


# ---------------------------------------------------------------- full workloads

def test_small_scan_workload():
    x = wl.small_scan()
    check_scan(x, "sum", True)
    check_scan(x, "sum", False)


def test_big_scan_workload_full_compare():
    """int32 exclusive sum, N = 2^28, values U{0..15}: every element compared."""
    x = wl.big_scan()
    check_scan(x, "sum", False)


def test_fp32_scan_workload():
    x = wl.fp32_scan()
    check_scan(x, "sum", True)


def test_max_scan_workload():
    x = wl.max_scan()
    check_scan(x, "max", True)
