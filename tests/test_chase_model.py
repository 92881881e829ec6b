"""Model of the chasing wave's group scan, on the CPU: why its float results repeat.

The wave that publishes tile prefixes scans a group of 64 tile totals with the
64-lane DPP scan of ls_device.hpp (row_shr 1, 2, 4, 8 inside rows of 16 lanes, then
lane 15 broadcast into rows 1 and 3 and lane 31 into rows 2 and 3; a lane whose
source is out of range receives the identity).  Lanes whose totals have not arrived
hold the identity, and the group is scanned again at every poll that finds more.
The claim: lane j's value depends only on lanes 0 .. j, through steps fixed by j,
so whatever a poll found, the prefixes it publishes carry exactly the bits of one
scan of the complete group.  This model replays the steps in float32 and checks
that, and that the claim is not vacuous (another association gives other bits)."""
import numpy as np
import pytest

F = np.float32


def add(a, b):
    return F(F(a) + F(b))


def dpp_wave_scan(v):
    """The six DPP steps on 64 float32 lanes (sum, identity +0.0)."""
    v = [F(x) for x in v]
    for s in (1, 2, 4, 8):  # inside rows of 16
        v = [add(v[l - s] if (l % 16) >= s else F(0.0), v[l]) for l in range(64)]
    # lane 15 of the row before into rows 1 and 3; rows 0 and 2 keep their value
    v = [add(v[16 * (l // 16) - 1], v[l]) if (l // 16) in (1, 3) else add(F(0.0), v[l])
         for l in range(64)]
    # lane 31 into rows 2 and 3
    v = [add(v[31], v[l]) if (l // 16) in (2, 3) else add(F(0.0), v[l]) for l in range(64)]
    return np.array(v, dtype=F)


def test_model_is_an_inclusive_scan():
    g = np.random.default_rng(1)
    x = g.integers(-1000, 1000, 64).astype(F)  # exact in float32
    assert np.array_equal(dpp_wave_scan(x), np.cumsum(x.astype(np.float64)).astype(F))


@pytest.mark.parametrize("seed", range(20))
def test_partial_groups_publish_the_full_groups_bits(seed):
    g = np.random.default_rng(100 + seed)
    x = (g.standard_normal(64) * 10.0 ** g.uniform(-3, 6, 64)).astype(F)
    base = F(g.standard_normal() * 1e4)  # the previous group's last prefix
    full = np.array([add(base, s) for s in dpp_wave_scan(x)], dtype=F)
    # polls that find the totals in stages: after each, lanes 0 .. k-1 hold totals
    ks = np.sort(g.choice(np.arange(1, 64), size=int(g.integers(1, 8)), replace=False)).tolist() + [64]
    published = np.full(64, np.nan, dtype=F)
    have = 0
    for k in ks:
        part = np.where(np.arange(64) < k, x, F(0.0)).astype(F)
        inc = np.array([add(base, s) for s in dpp_wave_scan(part)], dtype=F)
        published[have:k] = inc[have:k]
        have = k
    assert np.array_equal(published.view(np.uint32), full.view(np.uint32))


def test_another_association_gives_other_bits():
    """Windows that start where the previous poll stopped regroup the totals; with
    float32 totals of mixed magnitude that changes the bits."""
    g = np.random.default_rng(7)
    diffs = 0
    for _ in range(50):
        x = (g.standard_normal(64) * 10.0 ** g.uniform(-3, 6, 64)).astype(F)
        full = dpp_wave_scan(x)
        k = int(g.integers(8, 56))
        first = dpp_wave_scan(np.where(np.arange(64) < k, x, F(0.0)).astype(F))
        second = dpp_wave_scan(np.concatenate([x[k:], np.zeros(k, dtype=F)]))
        regrouped = np.concatenate([first[:k], [add(first[k - 1], s) for s in second[:64 - k]]]).astype(F)
        diffs += int(np.any(regrouped.view(np.uint32) != full.view(np.uint32)))
    assert diffs > 0
