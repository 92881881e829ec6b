"""scan_noalloc (the scan on the library's fixed per-GPU workspace) against the
scan entry points that take a caller's workspace, through the C ABI.

Each case calls scan_noalloc twice in a row on one stream, the second time on a
smaller input, and compares both results with scan_inclusive / scan_exclusive on
the same inputs: bit for bit (both run the same single-pass kernels, whose order
of combination depends only on n) and, for integers, with the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host

pytestmark = pytest.mark.gpu

SP_TILE = 28672
CASES = [("int32", "sum"), ("uint32", "xor"), ("int32", "max"), ("float32", "sum"),
         ("float32", "max"), ("uint32", "affine")]
# (first n, second n): several tiles and a ragged tail, then fewer tiles
SIZE_PAIRS = [(40 * SP_TILE + 13, 3 * SP_TILE + 5), (1_000_003, 777), (2 * SP_TILE, 1)]


def _reference(x, op, exclusive):
    fn = ps.scan_exclusive if exclusive else ps.scan_inclusive
    total = torch.empty(1, dtype=x.dtype, device=DEV)
    return fn(x, op, total=total), total


@pytest.mark.parametrize("n1,n2", SIZE_PAIRS)
@pytest.mark.parametrize("dtype,op", CASES)
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_noalloc_matches_workspace_scan(dtype, op, exclusive, n1, n2):
    print(f"scan_noalloc {dtype} {op} exclusive={exclusive} n={n1} then n={n2}", flush=True)
    for k, n in enumerate((n1, n2)):
        xh = wl.case(dtype, op, n, seed=9100 + 7 * k + n % 1000)
        x = to_dev(xh)
        out = torch.empty_like(x)
        total = torch.empty(1, dtype=x.dtype, device=DEV)
        ps.scan_noalloc(x, op, exclusive, out=out, total=total)
        got, got_total = to_host(out), to_host(total)
        ref_out, ref_total = _reference(x, op, exclusive)
        want, want_total = to_host(ref_out), to_host(ref_total)
        mism = np.flatnonzero(bits(got) != bits(want))
        assert mism.size == 0, f"call {k}: {mism.size} cells differ from the workspace scan, first {mism[0]}"
        assert bits(got_total)[0] == bits(want_total)[0], f"call {k}: totals differ"
        if dtype != "float32":
            ref = oracle.scan(xh, op, not exclusive)
            assert np.array_equal(bits(got), bits(ref.y)), f"call {k}: differs from the oracle"


def test_noalloc_largest_size_then_small():
    """At LS_SCAN_NOALLOC_MAX_N the fixed workspace still holds every tile's status."""
    n = ps.SCAN_NOALLOC_MAX_N
    print(f"scan_noalloc int32 sum exclusive n={n} then n=5", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(20260930)
    x = torch.randint(0, 16, (n,), dtype=torch.int32, device=DEV, generator=g)
    out = torch.empty_like(x)
    total = torch.empty(1, dtype=torch.int32, device=DEV)
    ps.scan_noalloc(x, "sum", True, out=out, total=total)
    want, want_total = _reference(x, "sum", True)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    assert torch.equal(total, want_total)
    del want, out
    xs = torch.tensor([3, 1, 4, 1, 5], dtype=torch.int32, device=DEV)
    got = to_host(ps.scan_noalloc(xs, "sum", True))
    assert got.tolist() == [0, 3, 4, 8, 9]


def test_noalloc_rejects_larger_than_max():
    x = torch.zeros(4, dtype=torch.int32, device=DEV)
    lib = ps.load_library()
    st = lib.scan_noalloc(x.data_ptr(), x.data_ptr(), ps.SCAN_NOALLOC_MAX_N + 1, 0, 0, 1, None, None)
    assert st == ps.LS_ERR_WORKSPACE
