"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds random-number recipes only -- none of the scan or compaction
arithmetic -- so that the CPU oracle and the HIP library are fed identical inputs
without either depending on the other.  Every generator is numpy PCG64
(``numpy.random.default_rng(seed)``), on the host.

Workloads (element counts and value distributions of the scan / compaction
workloads measured by this project):
  small_scan      int32 sum, inclusive + exclusive, N = 2^20, values U{0..9}
  big_scan        int32 exclusive sum, N = 2^28, values U{0..15}
  fp32_scan       float32 inclusive sum, N = 2^26, values U[-1, 1)
  max_scan        int32 inclusive max, N = 2^26, values U[-2^30, 2^30)
  compact         int32 stable compaction, N = 2^27, values U[0, 2^31),
                  predicate x < round(s * 2^31) for selectivity s in {1%, 50%, 99%}
  rows64          batched exclusive sum, 2^20 rows x 64 float32, values U[0, 1)
  rows1024        batched exclusive sum, 2^16 rows x 1024 int32, values U{0..9}
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20260925

SEEDS = {
    "small_scan": BASE_SEED + 0,
    "big_scan": BASE_SEED + 1,
    "fp32_scan": BASE_SEED + 2,
    "max_scan": BASE_SEED + 2,
    "compact": BASE_SEED + 3,
    "rows64": BASE_SEED + 4,
    "rows1024": BASE_SEED + 4,
}

SIZES = {
    "small_scan": 1 << 20,
    "big_scan": 1 << 28,
    "fp32_scan": 1 << 26,
    "max_scan": 1 << 26,
    "compact": 1 << 27,
    "rows64": (1 << 20, 64),
    "rows1024": (1 << 16, 1024),
}

SELECTIVITIES = (0.01, 0.50, 0.99)

# The 8-element worked example of the parallel prefix scan page (geek-doc.cn,
# section 一).
WORKED_EXAMPLE = np.array([3, 1, 4, 1, 5, 9, 2, 6], dtype=np.int32)


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def int_uniform(n, lo, hi_exclusive, seed, dtype=np.int32) -> np.ndarray:
    """n i.i.d. integers uniform in [lo, hi_exclusive), as dtype."""
    g = rng(seed)
    if hi_exclusive - 1 <= np.iinfo(np.int32).max and lo >= np.iinfo(np.int32).min:
        return g.integers(lo, hi_exclusive, size=n, dtype=np.int32).astype(dtype, copy=False)
    return g.integers(lo, hi_exclusive, size=n, dtype=np.int64).astype(dtype)


def f32_uniform(n, lo, hi, seed) -> np.ndarray:
    """n i.i.d. float32 uniform in [lo, hi): numpy's float32 random in [0, 1),
    scaled in float32 (for [-1, 1): r*2 - 1, exact in float32)."""
    g = rng(seed)
    r = g.random(size=n, dtype=np.float32)
    if lo == 0.0 and hi == 1.0:
        return r
    return (r * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def u32_bits(n, seed) -> np.ndarray:
    """n i.i.d. uniform 32-bit patterns (for xor and uint32 cases)."""
    g = rng(seed)
    return g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)


def threshold_for(selectivity: float) -> int:
    """Threshold t with P(x < t) = selectivity for x uniform in [0, 2^31)."""
    return int(round(selectivity * (1 << 31)))


# ---- the named workloads -------------------------------------------------

def small_scan(n=None):
    return int_uniform(n or SIZES["small_scan"], 0, 10, SEEDS["small_scan"])


def big_scan(n=None):
    return int_uniform(n or SIZES["big_scan"], 0, 16, SEEDS["big_scan"])


def fp32_scan(n=None):
    return f32_uniform(n or SIZES["fp32_scan"], -1.0, 1.0, SEEDS["fp32_scan"])


def max_scan(n=None):
    return int_uniform(n or SIZES["max_scan"], -(1 << 30), 1 << 30, SEEDS["max_scan"] + 100)


def compact_input(n=None):
    return int_uniform(n or SIZES["compact"], 0, 1 << 31, SEEDS["compact"])


def rows64(rows=None, cols=64):
    r = rows or SIZES["rows64"][0]
    return f32_uniform(r * cols, 0.0, 1.0, SEEDS["rows64"]).reshape(r, cols)


def rows1024(rows=None, cols=1024):
    r = rows or SIZES["rows1024"][0]
    return int_uniform(r * cols, 0, 10, SEEDS["rows1024"] + 100).reshape(r, cols)


def case(dtype: str, op: str, n: int, seed: int) -> np.ndarray:
    """A generic parity case: values chosen so each (dtype, op) is exercised
    over its interesting range (sums small enough to stay meaningful, max / min
    over signed/unsigned ranges, xor over full bit patterns, and / or that change
    at scattered places, odd factors for products and affine multipliers)."""
    if dtype == "float32":
        if op == "sum":
            return f32_uniform(n, -1.0, 1.0, seed)
        if op == "prod":
            # factors near +-1 keep long products finite and away from zero
            g = rng(seed)
            return (g.uniform(0.995, 1.005, n) * g.choice([-1.0, 1.0], n)).astype(np.float32)
        g = rng(seed)
        return (g.standard_normal(n) * 1e3).astype(np.float32)
    if op in ("and", "or"):
        # all ones (and) / all zeros (or) except a few words that clear / set one bit,
        # so the prefix changes at scattered places instead of collapsing at once
        g = rng(seed)
        x = np.full(n, 0xFFFFFFFF if op == "and" else 0, np.uint32)
        pos = g.choice(n, min(n, 64), replace=False) if n else np.zeros(0, np.int64)
        b = (np.uint32(1) << g.integers(0, 32, pos.size).astype(np.uint32)).astype(np.uint32)
        x[pos] = ~b if op == "and" else b
        return x.view(np.int32) if dtype == "int32" else x
    if op == "prod":
        x = u32_bits(n, seed) | np.uint32(1)  # odd factors: units mod 2^32, never 0
        return x.view(np.int32) if dtype == "int32" else x
    if op == "affine":
        return u32_bits(n, seed) | np.uint32(1 << 16)  # odd multipliers keep every map invertible
    if op == "sum":
        if dtype == "int32":
            return int_uniform(n, -1000, 1000, seed)
        return int_uniform(n, 0, 1 << 32, seed, dtype=np.uint32)
    if op in ("max", "min"):
        if dtype == "int32":
            return int_uniform(n, -(1 << 31), 1 << 31, seed, dtype=np.int32)
        return u32_bits(n, seed)
    if dtype == "int32":
        return u32_bits(n, seed).view(np.int32)
    return u32_bits(n, seed)
