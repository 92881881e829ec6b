"""Parity of the HIP radix sort (through the C ABI) with the CPU oracle's stable sort:
bit-exact keys and values (stability makes the result unique)."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host

pytestmark = pytest.mark.gpu

TILE = 1024  # keys per wave tile of the sort (a block tile is 8 of them)


def make_keys(dtype, n, seed, dup):
    rng = np.random.default_rng(seed)
    if dtype == "float32":
        k = (rng.standard_normal(n) * (10 if dup else 1e6)).astype(np.float32)
        if dup:
            k = np.round(k).astype(np.float32)
        k[::11] = -0.0
        k[5::13] = 0.0
        return k
    if dtype == "int32":
        hi = 20 if dup else 1 << 31
        return rng.integers(-hi, hi, n, dtype=np.int64).astype(np.int32)
    hi = 50 if dup else 1 << 32
    return rng.integers(0, hi, n, dtype=np.uint64).astype(np.uint32)


def check_sort(keys, with_values=True, inplace=False):
    vals = np.arange(keys.size, dtype=np.uint32) if with_values else None
    want_k, want_v = oracle.sort(keys, vals)
    kd = to_dev(keys)
    vd = to_dev(vals) if with_values else None
    if inplace:
        gk, gv = ps.radix_sort(kd, vd, out_keys=kd, out_values=vd)
    else:
        gk, gv = ps.radix_sort(kd, vd)
    got_k = to_host(gk)
    mism = np.flatnonzero(bits(got_k) != bits(want_k))
    assert mism.size == 0, f"{mism.size} key mismatches, first at {mism[0]}"
    if with_values:
        got_v = to_host(gv)
        mv = np.flatnonzero(got_v != want_v)
        assert mv.size == 0, f"{mv.size} value mismatches (stability), first at {mv[0]}"


@pytest.mark.parametrize("n", [1, 2, 3, 63, 64, 65, TILE - 1, TILE, TILE + 1, 4 * TILE + 3,
                               8 * TILE - 1, 8 * TILE, 8 * TILE + 1, 100_003, (1 << 20) + 7])
@pytest.mark.parametrize("dtype", ["int32", "uint32", "float32"])
@pytest.mark.parametrize("dup", [False, True], ids=["spread", "dups"])
def test_sort_matches_oracle(dtype, dup, n):
    check_sort(make_keys(dtype, n, seed=n + 1, dup=dup))


@pytest.mark.parametrize("dtype", ["int32", "uint32", "float32"])
def test_sort_keys_only_and_inplace(dtype):
    k = make_keys(dtype, 50_000, seed=4, dup=True)
    check_sort(k, with_values=False)
    check_sort(k, with_values=True, inplace=True)


def test_sort_special_floats():
    k = np.array([np.nan, 1.0, -np.nan, -0.0, 0.0, -np.inf, np.inf, -1.0] * 3000, np.float32)
    check_sort(k)


def test_sort_extreme_ints():
    k = np.array([0, -1, 2**31 - 1, -2**31, 1, -2**31, 2**31 - 1] * 5000, np.int32)
    check_sort(k)
    check_sort(k.view(np.uint32))


def test_sort_empty():
    k = torch.empty(0, dtype=torch.int32, device=DEV)
    gk, gv = ps.radix_sort(k)
    assert gk.numel() == 0 and gv is None


def test_sort_large():
    """2^24 uint32 keys with index values: full compare against the oracle."""
    k = wl.u32_bits(1 << 24, seed=99)
    check_sort(k)
