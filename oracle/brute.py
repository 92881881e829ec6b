"""Brute-force, definition-level scan and compaction in pure Python (tiny n only).

Test infrastructure: it pins the C oracle on tiny inputs.  Each output cell is
recomputed from scratch as a reduction over its whole prefix (O(n^2)), with
Python integers masked to 32 bits, so it shares neither the serial carried
accumulator nor any code with ``oracle.c``.

Definitions ([Scan3] = geek-doc.cn, parallel prefix scan page, section 一):
  inclusive  y[i] = x[0] (+) ... (+) x[i]
  exclusive  z[i] = x[0] (+) ... (+) x[i-1], z[0] = identity of (+)
  compaction keep x[i] iff pred(x[i]), in input order ([Scan3] 一, [SIMT3] 4.1)
"""
from __future__ import annotations

import functools
import math

M32 = 0xFFFFFFFF


def _signed(v: int) -> int:
    v &= M32
    return v - (1 << 32) if v & 0x80000000 else v


def _mat2_mul(m, n):
    """2x2 integer matrix product m @ n (lists of rows), entries mod 2^16."""
    return [[(m[r][0] * n[0][c] + m[r][1] * n[1][c]) & 0xFFFF for c in range(2)] for r in range(2)]


def _affine_to_mat(e):
    return [[(e >> 16) & 0xFFFF, e & 0xFFFF], [0, 1]]


def op_fn(dtype: str, op: str):
    """Binary operator on Python ints holding 32-bit patterns (int32/uint32),
    called as f(earlier, later)."""
    if op == "sum":
        return lambda a, b: (a + b) & M32
    if op == "xor":
        return lambda a, b: (a ^ b) & M32
    if op == "max":
        if dtype == "int32":
            return lambda a, b: a if _signed(a) > _signed(b) else b
        return lambda a, b: a if (a & M32) > (b & M32) else b
    if op == "min":
        if dtype == "int32":
            return lambda a, b: a if _signed(a) < _signed(b) else b
        return lambda a, b: a if (a & M32) < (b & M32) else b
    if op == "and":
        return lambda a, b: a & b & M32
    if op == "or":
        return lambda a, b: (a | b) & M32
    if op == "prod":
        return lambda a, b: (a * b) & M32
    if op == "affine" and dtype == "uint32":
        # the map v -> a v + b as the matrix [[a, b], [0, 1]]; the later map is
        # applied after the earlier one, so its matrix multiplies on the left
        def f(a, b):
            m = _mat2_mul(_affine_to_mat(b), _affine_to_mat(a))
            assert m[1] == [0, 1]
            return (m[0][0] << 16) | m[0][1]
        return f
    raise ValueError(op)


def identity(dtype: str, op: str) -> int:
    if op == "max":
        return 0x80000000 if dtype == "int32" else 0
    if op == "min":
        return 0x7FFFFFFF if dtype == "int32" else 0xFFFFFFFF
    if op == "and":
        return 0xFFFFFFFF
    if op == "prod":
        return 1
    if op == "affine":
        return 1 << 16
    return 0


def reduce_bits(bits, dtype, op):
    f = op_fn(dtype, op)
    return functools.reduce(f, bits, identity(dtype, op))


def inclusive_bits(bits, dtype, op):
    """bits: list of 32-bit patterns.  Each y[i] recomputed from x[0..i]."""
    return [reduce_bits(bits[: i + 1], dtype, op) for i in range(len(bits))]


def exclusive_bits(bits, dtype, op):
    return [reduce_bits(bits[:i], dtype, op) for i in range(len(bits))]


def fsum_inclusive(vals):
    """Float prefix sums, each cell the correctly rounded sum of its prefix."""
    return [math.fsum(vals[: i + 1]) for i in range(len(vals))]


def fsum_exclusive(vals):
    return [math.fsum(vals[:i]) for i in range(len(vals))]


_CMP = {
    "lt": lambda a, b: a < b,
    "le": lambda a, b: a <= b,
    "gt": lambda a, b: a > b,
    "ge": lambda a, b: a >= b,
    "eq": lambda a, b: a == b,
    "ne": lambda a, b: a != b,
}


def compact_values(vals, cmp, thr):
    """vals/thr: Python numbers already in their dtype's meaning."""
    f = _CMP[cmp]
    kept = [v for v in vals if f(v, thr)]
    return kept, len(kept)
