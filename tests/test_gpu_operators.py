"""Parity of the scans under the further operators (min, and, or, product and the
non-commutative affine-map composition) with the CPU oracle, through the C ABI.

Integer results and float min are compared bit for bit.  The float32 product is
compared with the oracle's double product under the relative bound of a product
of k float32 factors in any association, |gpu - ref| <= k * 2^-23 * |ref| (one
rounding of at most 2^-24 per multiplication, doubled for margin), k = i + 1.
The affine maps compose in order only if every combine in the library keeps its
left-right order: single pass (tile-local, wave, block and look-back combines),
both three-phase schemes, and all four block-level scans of the batched kernel."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host, ws_error_word

pytestmark = pytest.mark.gpu

TILE = 16384     # the three-phase schemes' tile; the deterministic single pass's is 2 * TILE
SP_TILE = 28672  # the single pass's tile
SIZES = [1, 2, 3, 63, 64, 65, 1023, 4096, 4097, TILE - 1, TILE, TILE + 1, 2 * TILE - 1, 2 * TILE + 1,
         3 * TILE + 7, 70 * TILE + 5, 300_003, SP_TILE - 1, SP_TILE + 1, 2 * SP_TILE + 1,
         66 * SP_TILE + 3]
COMBOS = [("int32", "min"), ("uint32", "min"), ("float32", "min"), ("int32", "and"),
          ("uint32", "and"), ("int32", "or"), ("uint32", "or"), ("int32", "prod"),
          ("uint32", "prod"), ("float32", "prod"), ("uint32", "affine")]


def assert_matches(got: np.ndarray, ref: oracle.ScanResult, dtype: str, op: str):
    if dtype == "float32" and op == "prod":
        g = np.asarray(got, np.float64).reshape(-1)
        r = np.asarray(ref.y, np.float64).reshape(-1)
        if r.size == 0:
            return
        cols = ref.y.shape[-1] if ref.y.ndim == 2 else r.size
        k = (np.arange(r.size) % cols) + 1.0
        err = np.abs(g - r)
        allowed = k * 2.0 ** -23 * np.abs(r) + 1e-30
        bad = np.flatnonzero(err > allowed)
        assert bad.size == 0, f"fp32 product off bound at {bad[0]}: {g[bad[0]]} vs {r[bad[0]]}"
    else:
        mism = np.flatnonzero(bits(got).reshape(-1) != bits(ref.y).reshape(-1))
        assert mism.size == 0, f"{mism.size} mismatches, first at {mism[0]}"


def check_scan(x: np.ndarray, op: str, inclusive: bool, scheme: str = "single_pass"):
    dtype = str(x.dtype)
    ref = oracle.scan(x, op, inclusive)
    xd = to_dev(x)
    total = torch.empty(1, dtype=xd.dtype, device=DEV)
    if scheme == "single_pass":
        fn = ps.scan_inclusive if inclusive else ps.scan_exclusive
        out = fn(xd, op, total=total)
        assert ws_error_word() == 0  # (a three-phase workspace holds tile totals, no header)
    else:
        out = ps.scan_ex(xd, op, inclusive, scheme, total=total)
    assert_matches(to_host(out), ref, dtype, op)
    if x.size:
        t = to_host(total)
        if dtype == "float32" and op == "prod":
            r = float(ref.total)
            assert abs(float(t[0]) - r) <= (x.size + 1) * 2.0 ** -23 * abs(r) + 1e-30
        else:
            assert bits(t)[0] == bits(np.array([ref.total], dtype=x.dtype))[0]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,op", COMBOS)
@pytest.mark.parametrize("inclusive", [True, False], ids=["incl", "excl"])
def test_operator_scan_matches_oracle(dtype, op, inclusive, n):
    check_scan(wl.case(dtype, op, n, seed=2000 + n), op, inclusive)


@pytest.mark.parametrize("scheme", ["reduce_then_scan", "scan_then_propagate"])
@pytest.mark.parametrize("dtype,op", COMBOS)
@pytest.mark.parametrize("n", [TILE + 1, 37 * TILE + 11, TILE * TILE + 3 * TILE + 5])
def test_operator_schemes_match_oracle(dtype, op, scheme, n):
    if n > 1_000_000 and op not in ("affine", "prod"):
        pytest.skip("the recursive totals scan is exercised by the non-commutative operators")
    x = wl.case(dtype, op, n, seed=3000 + n)
    check_scan(x, op, True, scheme)
    check_scan(x, op, False, scheme)


@pytest.mark.parametrize("dtype,op", COMBOS)
def test_operator_empty_gives_identity_total(dtype, op):
    tdt = {"int32": torch.int32, "uint32": torch.uint32, "float32": torch.float32}[dtype]
    x = torch.empty(0, dtype=tdt, device=DEV)
    total = torch.empty(1, dtype=tdt, device=DEV)
    ps.scan_exclusive(x, op, total=total)
    want = {("int32", "min"): 0x7FFFFFFF, ("uint32", "min"): 0xFFFFFFFF,
            ("float32", "min"): 0x7F800000, ("float32", "prod"): 0x3F800000,
            ("uint32", "affine"): 0x00010000}.get((dtype, op))
    if want is None:
        want = {"and": 0xFFFFFFFF, "or": 0, "prod": 1}[op]
    assert bits(to_host(total))[0] == want


def test_float_min_ties_keep_the_later_element():
    # -0 and +0 compare equal: the prefix must carry the bits of the later one
    x = np.tile(np.array([0.0, -0.0, 1.0, -0.0, 0.0, 0.0], np.float32), 5000)
    check_scan(x, "min", True)
    check_scan(x, "min", False)


@pytest.mark.parametrize("kind", ["wave_dpp", "hillis_steele", "hillis_steele_double", "blelloch"])
@pytest.mark.parametrize("cols", [3, 64, 65, 1024, 3000])
@pytest.mark.parametrize("dtype,op", COMBOS)
def test_operator_batched_matches_oracle(dtype, op, cols, kind):
    if cols <= 64 and kind != "wave_dpp":
        pytest.skip("rows of <= 64 columns always use the 16-lane row kernel")
    rows = max(2, min(200, 100_000 // cols)) + 1
    x = wl.case(dtype, op, rows * cols, seed=4000 + cols).reshape(rows, cols)
    for exclusive in (True, False):
        ref = oracle.batched(x, op, inclusive=not exclusive)
        out = ps.batched_row_scan_ex(to_dev(x), op, exclusive, kind)
        assert_matches(to_host(out), ref, dtype, op)


def test_affine_scan_at_workload_size():
    """2^26 affine maps: composing out of order anywhere across 4096 tiles shows."""
    x = wl.case("uint32", "affine", 1 << 26, seed=5)
    check_scan(x, "affine", True)
