"""Inputs past 2^31 elements, where 32-bit element indices would overflow, checked
by properties that hold at any size (closed forms, invariants and sampled cells that
the CPU oracle computes one by one), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import prefix_scan_stream_amd as ps
from gpu_util import DEV, bits, to_host, ws_error_word

pytestmark = pytest.mark.gpu

TILE = 16384
N = (1 << 31) + 3 * TILE + 7   # past 2^31, ragged tail: 8 GiB per int32 array


def _free_gib():
    free, _ = torch.cuda.mem_get_info(DEV)
    return free / 2**30


def test_scan_past_2e31_ones_and_iota():
    """Inclusive scan of ones is i + 1 (mod 2^32); exclusive scan of the index pattern
    i mod 2^32 is the closed form i (i - 1) / 2 mod 2^32, checked on sampled cells."""
    if _free_gib() < 20:
        pytest.skip("needs about 17 GiB of device memory")
    x = torch.ones(N, dtype=torch.int32, device=DEV)
    y = ps.scan_inclusive(x, "sum")
    assert ws_error_word() == 0
    rng = np.random.default_rng(1)
    idx = np.concatenate([rng.integers(0, N, 4000), [0, (1 << 31) - 1, 1 << 31, N - 1]])
    got = to_host(y[torch.from_numpy(idx).to(DEV)]).view(np.uint32)
    assert np.array_equal(got, ((idx + 1) & 0xFFFFFFFF).astype(np.uint32))
    del y
    xi = torch.arange(N, dtype=torch.int64, device=DEV).to(torch.int32)   # i mod 2^32 (wraps)
    z = ps.scan_exclusive(xi, "sum")
    i = idx.astype(object)
    want = np.array([(v * (v - 1) // 2) & 0xFFFFFFFF for v in i], np.uint32)
    assert np.array_equal(to_host(z[torch.from_numpy(idx).to(DEV)]).view(np.uint32), want)


def test_compaction_past_2e31():
    """Keep every element whose value is below 5 of the pattern i mod 7: the count and
    sampled kept values follow in closed form."""
    if _free_gib() < 20:
        pytest.skip("needs about 17 GiB of device memory")
    x = (torch.arange(N, dtype=torch.int64, device=DEV) % 7).to(torch.int32)
    out, count = ps.compact_if(x, "lt", 5)
    c = int(to_host(count)[0])
    assert c == (N // 7) * 5 + min(N % 7, 5)
    rng = np.random.default_rng(2)
    # the last kept elements come from input positions past 2^31
    k = np.concatenate([rng.integers(0, c, 3000), [0, c - 1], c - 1 - np.arange(1, 2000)])
    # the k-th kept element: 5 kept per 7, so it is the value k mod 5
    assert np.array_equal(to_host(out[torch.from_numpy(k).to(DEV)]), (k % 5).astype(np.int32))


def test_segmented_past_2e31():
    """Segments of length 1000 over ones: the inclusive value at i is i mod 1000 + 1."""
    if _free_gib() < 25:
        pytest.skip("needs about 20 GiB of device memory")
    x = torch.ones(N, dtype=torch.int32, device=DEV)
    heads = (torch.arange(N, dtype=torch.int64, device=DEV) % 1000 == 0).to(torch.uint8)
    y = ps.segmented_scan(x, "sum", False, heads=heads)
    rng = np.random.default_rng(3)
    idx = np.concatenate([rng.integers(0, N, 4000), [N - 1, (1 << 31)]])
    assert np.array_equal(to_host(y[torch.from_numpy(idx).to(DEV)]), (idx % 1000 + 1).astype(np.int32))


def test_sampled_cells_of_a_random_2e31_scan():
    """Random values: sampled output cells against the oracle's serial scan of the
    whole input (the oracle finishes 2^31 cells in a few seconds)."""
    if _free_gib() < 20:
        pytest.skip("needs about 17 GiB of device memory")
    rng = np.random.default_rng(4)
    xh = rng.integers(0, 16, N, dtype=np.int32)
    ref = oracle.scan(xh, "sum", False).y
    y = to_host(ps.scan_exclusive(torch.from_numpy(xh).to(DEV), "sum"))
    idx = np.concatenate([rng.integers(0, N, 100000), [0, N - 1]])
    assert np.array_equal(bits(y[idx]), bits(ref[idx]))
    assert np.array_equal(y[-TILE:], ref[-TILE:])


def test_sort_past_2e31():
    """2^31 + 5 random uint32 keys with their positions as values: the keys come out
    non-decreasing, keys and values are the same multisets (sum and xor), values
    follow their keys on sampled cells, and ties keep their input order."""
    if _free_gib() < 60:
        pytest.skip("needs about 50 GiB of device memory")
    n = (1 << 31) + 5
    g = torch.Generator(device=DEV).manual_seed(5)
    keys = torch.randint(0, 1 << 20, (n,), dtype=torch.int32, device=DEV, generator=g).to(torch.uint32)
    vals = torch.arange(n, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.uint32)
    sk, sv = ps.radix_sort(keys, vals)
    step = 1 << 28
    prev = None
    for a in range(0, n, step):
        c = sk[a:a + step].to(torch.int64)
        if prev is not None:
            assert int(c[0]) >= prev
        assert bool((c[1:] >= c[:-1]).all())
        prev = int(c[-1])
    assert int(sk.to(torch.int64).sum()) == int(keys.to(torch.int64).sum())
    assert int(sv.to(torch.int64).sum()) == n * (n - 1) // 2
    rng = np.random.default_rng(6)
    idx = torch.from_numpy(np.concatenate([rng.integers(0, n, 20000), [n - 1]])).to(DEV)
    v = sv.view(torch.int32)[idx].to(torch.int64) & 0xFFFFFFFF      # uint32 positions
    assert bool((keys.view(torch.int32)[v] == sk.view(torch.int32)[idx]).all())
    # ties keep input order: among equal keys the values (input positions) increase
    same = sk[1:step] == sk[:step - 1]
    assert bool((sv[1:step].to(torch.int64)[same] > sv[:step - 1].to(torch.int64)[same]).all())
