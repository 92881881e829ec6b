"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with something other than itself: values the pages print (fixtures under
tests/golden/, each with its citation), closed forms, invariants, numpy library
routines that reduce to the same definition, and brute force over tiny inputs.
They are written as plain functions so the same list can be run against copies of
the oracle with a planted mistake (tests/test_oracle_mutants.py).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

from conftest import load_golden
from oracle import brute

INT_DTYPES = ("int32", "uint32")
OPS = ("sum", "max", "xor", "min", "and", "or", "prod", "affine")
FLOAT_OPS = ("sum", "max", "min", "prod")


def _defined(dtype, op):
    if dtype == "float32":
        return op in FLOAT_OPS
    return op != "affine" or dtype == "uint32"
M32 = 0xFFFFFFFF


def _bits(a):
    return [int(v) & M32 for v in np.asarray(a).view(np.uint32).tolist()]


def _ident(dtype, op):
    return brute.identity(dtype, op)


# ---------------------------------------------------------------- page values

def pin_worked_example_scan(orc):
    g = load_golden("worked_example.txt")
    x = np.array(g["x"], np.int32)
    inc = orc.scan(x, "sum", True)
    exc = orc.scan(x, "sum", False)
    assert inc.y.tolist() == g["inclusive"]
    assert exc.y.tolist() == g["exclusive"]
    assert int(inc.total) == g["total"][0] and int(exc.total) == g["total"][0]
    # the same example through the float path (exact: small integers)
    xf = x.astype(np.float32)
    fi = orc.scan(xf, "sum", True)
    fe = orc.scan(xf, "sum", False)
    assert fi.y.tolist() == [float(v) for v in g["inclusive"]]
    assert fe.y.tolist() == [float(v) for v in g["exclusive"]]
    # and as uint32
    assert orc.scan(x.view(np.uint32), "sum", False).y.tolist() == g["exclusive"]


def pin_worked_example_compaction(orc):
    g = load_golden("worked_example.txt")
    x = np.array(g["x"], np.int32)
    cmp, thr = g["predicate"][0], g["predicate"][1]
    for via in (False, True):
        out, count = orc.compact(x, cmp, thr, via_scan=via)
        assert out.tolist() == g["compacted"]
        assert count == g["count"][0]
    # the flags and their exclusive scan, as printed
    flags = np.array([1 if v > thr else 0 for v in g["x"]], np.int32)
    assert flags.tolist() == g["flags"]
    assert orc.scan(flags, "sum", False).y.tolist() == g["flags_exclusive"]


def pin_two_block_decomposition(orc):
    g = load_golden("two_block.txt")
    x = np.array(g["x"], np.int32)
    b = g["block_size"][0]
    blocks = [x[i:i + b] for i in range(0, len(x), b)]
    totals = [int(orc.scan(blk, "sum", True).total) for blk in blocks]
    assert totals == g["block_totals"]
    offsets = orc.scan(np.array(totals, np.int32), "sum", False).y.tolist()
    assert offsets == g["block_offsets"]
    local = orc.scan(blocks[1], "sum", False).y
    assert local.tolist() == g["block1_local_exclusive"]
    glob = (local + offsets[1]).tolist()
    assert glob == g["block1_global_exclusive"]
    assert orc.scan(x, "sum", False).y[b:].tolist() == glob


# ---------------------------------------------------------------- invariants

def pin_inclusive_exclusive_relation(orc):
    """z[0] = identity, z[i] = y[i-1], total = y[n-1] = z[n-1] (+) x[n-1]."""
    rng = np.random.default_rng(11)
    for dtype in INT_DTYPES:
        for op in OPS:
            if not _defined(dtype, op):
                continue
            for n in (1, 2, 7, 100):
                x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
                x = x.view(np.int32) if dtype == "int32" else x
                inc = orc.scan(x, op, True)
                exc = orc.scan(x, op, False)
                yb, zb = _bits(inc.y), _bits(exc.y)
                assert zb[0] == _ident(dtype, op)
                assert zb[1:] == yb[:-1]
                f = brute.op_fn(dtype, op)
                tb = int(np.array([inc.total]).view(np.uint32)[0])
                assert tb == yb[-1] == f(zb[-1], _bits(x)[-1])
                assert int(np.array([exc.total]).view(np.uint32)[0]) == tb


def pin_empty_input(orc):
    for dtype in INT_DTYPES + ("float32",):
        for op in OPS:
            if not _defined(dtype, op):
                continue
            x = np.zeros(0, dtype)
            for inc in (True, False):
                r = orc.scan(x, op, inc)
                assert r.y.size == 0
                if dtype != "float32":
                    assert int(np.array([r.total]).view(np.uint32)[0]) == _ident(dtype, op)
    out, c = orc.compact(np.zeros(0, np.int32), "lt", 5)
    assert c == 0 and out.size == 0


# ---------------------------------------------------------------- closed forms

def pin_closed_forms_sum(orc):
    n = 100_003  # n(n+1)/2 > 2^32: exercises the mod-2^32 wrap
    ones = np.ones(n, np.int32)
    assert np.array_equal(orc.scan(ones, "sum", True).y, np.arange(1, n + 1, dtype=np.int32))
    assert np.array_equal(orc.scan(ones, "sum", False).y, np.arange(0, n, dtype=np.int32))
    iota = np.arange(n, dtype=np.uint32)
    i = np.arange(n, dtype=np.uint64)
    want = ((i * (i + 1) // 2) & M32).astype(np.uint32)
    assert np.array_equal(orc.scan(iota, "sum", True).y, want)
    assert np.array_equal(orc.scan(iota.view(np.int32), "sum", True).y.view(np.uint32), want)
    # exclusive of iota: i(i-1)/2
    want_e = ((i * (i - 1) // 2) & M32).astype(np.uint32)
    want_e[0] = 0
    assert np.array_equal(orc.scan(iota, "sum", False).y, want_e)


def pin_closed_forms_xor(orc):
    """xor of 0..k is k, 1, k+1, 0 for k mod 4 = 0, 1, 2, 3."""
    n = 5000
    iota = np.arange(n, dtype=np.uint32)
    y = orc.scan(iota, "xor", True).y.tolist()
    for k in range(n):
        assert y[k] == [k, 1, k + 1, 0][k % 4]
    # self-inverse: x xor-scanned twice from a shifted copy recovers x
    z = orc.scan(iota, "xor", False).y
    assert np.array_equal(z ^ orc.scan(iota, "xor", True).y, iota)


def pin_closed_forms_max(orc):
    asc = np.arange(-500, 500, dtype=np.int32)
    assert np.array_equal(orc.scan(asc, "max", True).y, asc)
    desc = asc[::-1].copy()
    assert np.array_equal(orc.scan(desc, "max", True).y, np.full_like(desc, desc[0]))
    e = orc.scan(desc, "max", False).y
    assert int(e[0]) == -(1 << 31) and np.all(e[1:] == desc[0])
    # signed vs unsigned: 0xFFFFFFFF is -1 as int32 but the largest uint32
    x = np.array([5, -1, 3], np.int32)
    assert orc.scan(x, "max", True).y.tolist() == [5, 5, 5]
    assert orc.scan(x.view(np.uint32), "max", True).y.tolist() == [5, 0xFFFFFFFF, 0xFFFFFFFF]
    # float max: ascending / descending, exclusive starts at -inf
    f = np.linspace(-3, 3, 101).astype(np.float32)
    assert np.array_equal(orc.scan(f, "max", True).y, f)
    fd = f[::-1].copy()
    assert np.array_equal(orc.scan(fd, "max", True).y, np.full_like(fd, fd[0]))
    fe = orc.scan(fd, "max", False).y
    assert np.isneginf(fe[0]) and np.all(fe[1:] == fd[0])


def pin_float_max_tie_rule(orc):
    """Ties keep the right operand: the prefix carries the bits of the right-most of
    its largest elements (seen through +0 / -0)."""
    x = np.array([0.0, -0.0, 1.0, -0.0, 0.0, -0.0], np.float32)
    y = orc.scan(x, "max", True).y
    assert _bits(y) == _bits(np.array([0.0, -0.0, 1.0, 1.0, 1.0, 1.0], np.float32))
    x2 = np.array([-0.0, 0.0, -0.0], np.float32)
    assert _bits(orc.scan(x2, "max", True).y) == _bits(x2)


# ---------------------------------------------------------------- library routines

def pin_numpy_cumulative(orc):
    rng = np.random.default_rng(7)
    n = 20_000
    xi = rng.integers(-(1 << 31), 1 << 31, n, dtype=np.int64).astype(np.int32)
    xu = xi.view(np.uint32)
    cs = (np.cumsum(xu.astype(np.uint64)) & M32).astype(np.uint32)
    assert np.array_equal(orc.scan(xi, "sum", True).y.view(np.uint32), cs)
    assert np.array_equal(orc.scan(xu, "sum", True).y, cs)
    assert np.array_equal(orc.scan(xi, "max", True).y, np.maximum.accumulate(xi))
    assert np.array_equal(orc.scan(xu, "max", True).y, np.maximum.accumulate(xu))
    assert np.array_equal(orc.scan(xu, "xor", True).y, np.bitwise_xor.accumulate(xu))
    xf = (rng.standard_normal(n) * 100).astype(np.float32)
    assert np.array_equal(orc.scan(xf, "max", True).y, np.maximum.accumulate(xf))


def pin_fp32_sum_exact_and_fsum(orc):
    """Integer-valued float32 data with partial sums < 2^24 is summed exactly in any
    order; general float data matches correctly rounded prefix sums (math.fsum)."""
    rng = np.random.default_rng(5)
    xi = rng.integers(-50, 50, 3000).astype(np.float32)
    inc = orc.scan(xi, "sum", True)
    exc = orc.scan(xi, "sum", False)
    ci = np.cumsum(xi.astype(np.int64))
    assert np.array_equal(inc.y, ci.astype(np.float64))
    assert exc.y[0] == 0.0 and np.array_equal(exc.y[1:], ci[:-1].astype(np.float64))
    assert np.array_equal(inc.bound, np.cumsum(np.abs(xi.astype(np.int64))).astype(np.float64))
    assert np.array_equal(exc.bound, inc.bound)
    assert inc.total == exc.total == float(ci[-1])
    xf = (rng.random(300) * 2 - 1).astype(np.float32)
    vals = [float(v) for v in xf]
    fi = brute.fsum_inclusive(vals)
    fe = brute.fsum_exclusive(vals)
    ri = orc.scan(xf, "sum", True).y
    re = orc.scan(xf, "sum", False).y
    for k in range(len(vals)):
        assert abs(ri[k] - fi[k]) <= 1e-12 * (1 + abs(fi[k]))
        assert abs(re[k] - fe[k]) <= 1e-12 * (1 + abs(fe[k]))
    assert np.allclose(orc.scan(xf, "sum", True).bound,
                       np.cumsum(np.abs(xf.astype(np.float64))), rtol=1e-14, atol=0)


# ---------------------------------------------------------------- brute force

def pin_brute_force_random(orc):
    rng = np.random.default_rng(3)
    for dtype in INT_DTYPES:
        for op in OPS:
            if not _defined(dtype, op):
                continue
            for n in list(range(1, 17)) + [31, 64]:
                x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
                if op == "sum" and rng.random() < 0.5:
                    x = rng.integers(0, 10, n).astype(np.uint32)
                x = x.view(np.int32) if dtype == "int32" else x
                b = _bits(x)
                assert _bits(orc.scan(x, op, True).y) == brute.inclusive_bits(b, dtype, op)
                assert _bits(orc.scan(x, op, False).y) == brute.exclusive_bits(b, dtype, op)


def pin_brute_force_exhaustive_tiny(orc):
    alphabet = [0, 1, 2, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFF]
    for dtype in INT_DTYPES:
        for op in OPS:
            if not _defined(dtype, op):
                continue
            for n in range(1, 5):
                for combo in itertools.product(alphabet, repeat=n):
                    x = np.array(combo, np.uint32)
                    x = x.view(np.int32) if dtype == "int32" else x
                    b = list(combo)
                    assert _bits(orc.scan(x, op, True).y) == brute.inclusive_bits(b, dtype, op)
                    assert _bits(orc.scan(x, op, False).y) == brute.exclusive_bits(b, dtype, op)


def pin_more_operators_numpy(orc):
    """min / and / or / product against numpy's own accumulations ([Blog2] 3.3)."""
    rng = np.random.default_rng(29)
    for n in (1, 2, 33, 1000):
        xu = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        xi = xu.view(np.int32)
        assert np.array_equal(orc.scan(xu, "min", True).y, np.minimum.accumulate(xu))
        assert np.array_equal(orc.scan(xi, "min", True).y, np.minimum.accumulate(xi))
        assert np.array_equal(orc.scan(xu, "and", True).y, np.bitwise_and.accumulate(xu))
        assert np.array_equal(orc.scan(xu, "or", True).y, np.bitwise_or.accumulate(xu))
        assert np.array_equal(orc.scan(xu, "prod", True).y, np.multiply.accumulate(xu, dtype=np.uint32))
        assert np.array_equal(orc.scan(xi, "prod", True).y.view(np.uint32),
                              np.multiply.accumulate(xu, dtype=np.uint32))
        xf = rng.standard_normal(n).astype(np.float32)
        assert np.array_equal(orc.scan(xf, "min", True).y, np.minimum.accumulate(xf))


def pin_more_operators_closed_forms(orc):
    n = 200
    i = np.arange(n)
    desc = (1000 - i).astype(np.int32)
    assert np.array_equal(orc.scan(desc, "min", True).y, desc)
    assert np.all(orc.scan(desc[::-1].copy(), "min", True).y == desc[-1])
    threes = np.full(n, 3, np.uint32)
    assert _bits(orc.scan(threes, "prod", True).y) == [pow(3, k + 1, 1 << 32) for k in range(n)]
    assert _bits(orc.scan(threes, "prod", False).y) == [pow(3, k, 1 << 32) for k in range(n)]
    bit = np.array([1 << (k % 32) for k in range(n)], np.uint32)
    assert _bits(orc.scan(bit, "or", True).y) == [(1 << min(k + 1, 32)) - 1 for k in range(n)]
    clear = ~bit
    assert _bits(orc.scan(clear, "and", True).y) == [M32 ^ ((1 << min(k + 1, 32)) - 1)
                                                    for k in range(n)]
    ones = np.full(n, (1 << 16) | 1, np.uint32)            # v -> v + 1
    assert _bits(orc.scan(ones, "affine", True).y) == [(1 << 16) | ((k + 1) & 0xFFFF)
                                                      for k in range(n)]
    tri = np.full(n, 3 << 16, np.uint32)                   # v -> 3 v
    assert _bits(orc.scan(tri, "affine", True).y) == [pow(3, k + 1, 1 << 16) << 16 for k in range(n)]
    # float min: the right-most of equal minima, and the +inf identity
    f = np.array([0.0, -0.0, 1.0, -0.0, 0.0], np.float32)
    assert _bits(orc.scan(f, "min", True).y) == _bits(np.array([0.0, -0.0, -0.0, -0.0, 0.0],
                                                               np.float32))
    assert _bits(orc.scan(f, "min", False).y[:1]) == [0x7F800000]


def pin_affine_maps_compose_in_order(orc):
    """Scanning affine maps ([Scan3] 三: a non-commutative operator keeps its left-right
    order): y[i] applied to v equals applying x[0], x[1], ..., x[i] to v one after the
    other, computed here by plain evaluation, without composing anything."""
    rng = np.random.default_rng(31)
    for n in (1, 2, 5, 64, 300):
        x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        y = _bits(orc.scan(x, "affine", True).y)
        z = _bits(orc.scan(x, "affine", False).y)
        for v0 in (0, 1, 12345, 65535):
            v = v0
            for k in range(n):
                assert ((z[k] >> 16) * v0 + (z[k] & 0xFFFF)) & 0xFFFF == v
                a, b = int(x[k]) >> 16, int(x[k]) & 0xFFFF
                v = (a * v + b) & 0xFFFF
                assert ((y[k] >> 16) * v0 + (y[k] & 0xFFFF)) & 0xFFFF == v


def pin_float_product(orc):
    """Products of powers of two are exact in any order; other products match the
    exact rational product within the double's own rounding."""
    import fractions
    rng = np.random.default_rng(37)
    p2 = np.ldexp(1.0, rng.integers(-3, 4, 100)).astype(np.float32) * rng.choice([-1, 1], 100)
    want, acc = [], 1.0
    for v in p2.tolist():
        acc *= v
        want.append(acc)
    assert orc.scan(p2.astype(np.float32), "prod", True).y.tolist() == want
    xs = rng.uniform(0.5, 2.0, 200).astype(np.float32)
    y = orc.scan(xs, "prod", True).y
    exact = fractions.Fraction(1)
    for k, v in enumerate(xs.tolist()):
        exact *= fractions.Fraction(v)
        assert abs(fractions.Fraction(float(y[k])) - exact) <= exact * (k + 1) * fractions.Fraction(1, 2**52)
    assert orc.scan(xs, "prod", False).y[0] == 1.0


def _exact_products(vals, starts, inclusive):
    """Running products restarted where starts[i] is true, in exact rationals."""
    import fractions
    out, acc = [], fractions.Fraction(1)
    for v, s in zip(vals, starts):
        if s:
            acc = fractions.Fraction(1)
        if inclusive:
            acc *= fractions.Fraction(v)
            out.append(float(acc))
        else:
            out.append(float(acc))
            acc *= fractions.Fraction(v)
    return out


def pin_float_product_segmented_and_batched(orc):
    """Float products restart at every segment head and every row start ([Blog2]
    §7.2; the product operator of §3.3).  Signed powers of two multiply exactly in
    any order, so the expected prefixes are exact rationals computed here, segment
    by segment and row by row, with nothing taken from the oracle."""
    rng = np.random.default_rng(53)
    n = 400
    x = (np.ldexp(1.0, rng.integers(-3, 4, n)) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    heads = (rng.random(n) < 0.12).astype(np.uint8)
    heads[0] = 0  # element 0 starts a segment whether or not it is flagged
    heads[n - 1] = 1  # a one-element segment at the end
    starts = [i == 0 or bool(heads[i]) for i in range(n)]
    vals = x.tolist()
    for inc in (True, False):
        assert orc.segmented(x, "prod", inc, heads=heads).y.tolist() == _exact_products(vals, starts, inc)
        offs = np.concatenate([np.flatnonzero(starts), [n]]).astype(np.int64)
        assert orc.segmented(x, "prod", inc, offsets=offs).y.tolist() == _exact_products(vals, starts, inc)
    rows, cols = 8, 50
    xr = x.reshape(rows, cols)
    row_starts = [j == 0 for j in range(cols)]
    for inc in (True, False):
        y = orc.batched(xr, "prod", inc).y
        assert y.shape == (rows, cols)
        for r in range(rows):
            assert y[r].tolist() == _exact_products(xr[r].tolist(), row_starts, inc), f"row {r}"


# ---------------------------------------------------------------- segmented scan

def _brute_segmented(bits, heads, dtype, op, inclusive):
    """Each cell recomputed from its own segment: the last head at or before i."""
    f = brute.op_fn(dtype, op)
    out = []
    for i in range(len(bits)):
        start = max(j for j in range(i + 1) if j == 0 or heads[j])
        seg = bits[start:i + 1] if inclusive else bits[start:i]
        acc = brute.identity(dtype, op)
        for v in seg:
            acc = f(acc, v)
        out.append(acc)
    return out


def pin_segmented_special_cases(orc):
    """Uniform segments are the batched rows; one segment is the plain scan; a head
    on every element leaves x (inclusive) or the identity (exclusive)."""
    rng = np.random.default_rng(41)
    for dtype, op in (("int32", "sum"), ("uint32", "xor"), ("int32", "max"), ("uint32", "affine"),
                      ("int32", "prod"), ("float32", "max"), ("float32", "min"), ("float32", "prod")):
        rows, cols = 7, 13
        x = wl_case(rng, dtype, op, rows * cols)
        if (dtype, op) == ("float32", "prod"):
            x = (x / np.float32(16)).astype(np.float32)  # keep the products of a row in range
        heads = np.zeros(rows * cols, np.uint8)
        heads[::cols] = 1
        for inc in (True, False):
            seg = orc.segmented(x, op, inc, heads=heads).y
            bat = orc.batched(x.reshape(rows, cols), op, inc).y.reshape(-1)
            assert _bits(seg) == _bits(bat)
            one = orc.segmented(x, op, inc, heads=np.zeros(rows * cols, np.uint8)).y
            assert _bits(one) == _bits(orc.scan(x, op, inc).y)
        every = orc.segmented(x, op, True, heads=np.ones(rows * cols, np.uint8)).y
        ex = orc.segmented(x, op, False, heads=np.full(rows * cols, 7, np.uint8)).y
        if (dtype, op) == ("float32", "prod"):  # float products are carried in double
            assert every.tolist() == [float(v) for v in x.tolist()]
            assert all(v == 1.0 for v in ex.tolist())
            continue
        assert _bits(every) == _bits(x)
        want = _ident(dtype, op) if dtype != "float32" else {"max": 0xFF800000, "min": 0x7F800000}[op]
        assert all(b == want for b in _bits(ex))


def wl_case(rng, dtype, op, n):
    if dtype == "float32":
        return rng.integers(-50, 50, n).astype(np.float32)
    x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    if op == "affine":
        x |= np.uint32(1 << 16)
    return x.view(np.int32) if dtype == "int32" else x


def pin_segmented_brute_force(orc):
    rng = np.random.default_rng(43)
    for dtype in INT_DTYPES:
        for op in OPS:
            if not _defined(dtype, op):
                continue
            for n in (1, 2, 5, 17, 40):
                x = wl_case(rng, dtype, op, n)
                heads = (rng.random(n) < 0.3).astype(np.uint8)
                for inc in (True, False):
                    got = _bits(orc.segmented(x, op, inc, heads=heads).y)
                    assert got == _brute_segmented(_bits(x), heads.tolist(), dtype, op, inc)


def pin_segmented_numpy_and_offsets(orc):
    """int32 sums against numpy (prefix sums minus the sum before each segment), float
    sums of small integers exactly, and offsets against the equivalent head flags."""
    rng = np.random.default_rng(47)
    n = 5000
    x = rng.integers(-1000, 1000, n).astype(np.int32)
    starts = np.unique(np.concatenate([[0], rng.integers(0, n, 300)]))
    heads = np.zeros(n, np.uint8)
    heads[starts] = 1
    c = np.cumsum(x.astype(np.int64))
    seg_of = np.cumsum(heads) - 1                     # segment index of each element
    before = np.concatenate([[0], c])[starts][seg_of]  # sum of everything before the segment
    assert np.array_equal(orc.segmented(x, "sum", True, heads=heads).y.astype(np.int64), c - before)
    assert np.array_equal(orc.segmented(x, "sum", False, heads=heads).y.astype(np.int64),
                          c - x - before)
    xf = x.astype(np.float32)
    r = orc.segmented(xf, "sum", True, heads=heads)
    assert np.array_equal(r.y, (c - before).astype(np.float64))
    assert np.all(r.bound >= np.abs(r.y))
    # offsets, with empty segments (repeated offsets) and a final empty segment
    offs = np.concatenate([[0], np.sort(rng.integers(0, n, 400)), [n, n]]).astype(np.int64)
    h2 = np.zeros(n, np.uint8)
    h2[offs[:-1][offs[:-1] < n]] = 1
    for op in ("sum", "max", "xor"):
        for inc in (True, False):
            a = orc.segmented(x, op, inc, offsets=offs).y
            b = orc.segmented(x, op, inc, heads=h2).y
            assert np.array_equal(a, b)
    # worked example: segments [3 1 4] [1 5] [9 2 6], the last one not empty
    xe = np.array([3, 1, 4, 1, 5, 9, 2, 6], np.int32)
    offe = np.array([0, 3, 5, 8], np.int64)
    assert orc.segmented(xe, "sum", True, offsets=offe).y.tolist() == [3, 4, 8, 1, 6, 9, 11, 17]
    assert orc.segmented(xe, "sum", False, offsets=offe).y.tolist() == [0, 3, 4, 0, 1, 0, 9, 11]
    # float max / min ties: the later of equal elements (-0 against +0) is kept
    z = np.array([0.0, -0.0, 0.0, -0.0, -0.0, 0.0], np.float32)
    hz = np.array([1, 0, 0, 1, 0, 0], np.uint8)
    for op in ("max", "min"):
        assert _bits(orc.segmented(z, op, True, heads=hz).y) == _bits(z)
    for bad in ([1, n], [0, n - 1], [0, 10, 5, n]):
        try:
            orc.segmented(x, "sum", True, offsets=np.array(bad, np.int64))
        except ValueError:
            continue
        raise AssertionError(f"offsets {bad} were accepted")


def pin_compaction_brute_and_numpy(orc):
    rng = np.random.default_rng(9)
    cmps = ("lt", "le", "gt", "ge", "eq", "ne")
    for dtype in ("int32", "uint32", "float32"):
        for n in (1, 5, 17, 64, 1000):
            if dtype == "float32":
                x = rng.integers(-4, 5, n).astype(np.float32)
                thr = np.float32(1.0)
            elif dtype == "int32":
                x = rng.integers(-4, 5, n).astype(np.int32)
                thr = np.int32(1)
            else:
                x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
                x[::3] = 0x7FFFFFFF
                thr = np.uint32(0x7FFFFFFF)
            vals = x.tolist()
            for cmp in cmps:
                want, wc = brute.compact_values(vals, cmp, thr.item())
                for via in (False, True):
                    out, c = orc.compact(x, cmp, thr, via_scan=via)
                    assert c == wc and out.tolist() == want
    # numpy boolean mask at a larger size, selectivities 0, 50 %, 100 %
    x = rng.integers(0, 1 << 31, 200_000, dtype=np.int64).astype(np.int32)
    for thr in (0, 1 << 30, (1 << 31) - 1):
        out, c = orc.compact(x, "lt", thr)
        want = x[x < thr]
        assert c == want.size and np.array_equal(out, want)
    out, c = orc.compact(x, "ge", 0)  # everything kept: an exact copy
    assert c == x.size and np.array_equal(out, x)
    # stability of the payload bits: -0.0 and +0.0 are equal under ==, both kept in order
    xz = np.array([0.0, -0.0, 1.0, -0.0], np.float32)
    out, c = orc.compact(xz, "eq", np.float32(0.0))
    assert c == 3 and _bits(out) == _bits(np.array([0.0, -0.0, -0.0], np.float32))
    # NaN is unordered: never < or ==, always !=
    xn = np.array([np.nan, 1.0, np.nan], np.float32)
    assert orc.compact(xn, "lt", np.float32(5.0))[1] == 1
    assert orc.compact(xn, "ne", np.float32(1.0))[1] == 2


def pin_batched_rows(orc):
    rng = np.random.default_rng(13)
    x = rng.integers(0, 10, (37, 64)).astype(np.int32)
    y = orc.batched(x, "sum", False).y
    want = np.cumsum(x, axis=1) - x
    assert np.array_equal(y, want.astype(np.int32))
    assert np.all(y[:, 0] == 0)  # no carry from the previous row
    yi = orc.batched(x, "sum", True).y
    assert np.array_equal(yi, np.cumsum(x, axis=1).astype(np.int32))
    xm = rng.integers(-100, 100, (9, 33)).astype(np.int32)
    assert np.array_equal(orc.batched(xm, "max", True).y, np.maximum.accumulate(xm, axis=1))
    xf = rng.random((5, 64)).astype(np.float32)
    r = orc.batched(xf, "sum", False)
    for row in range(5):
        fe = brute.fsum_exclusive([float(v) for v in xf[row]])
        assert max(abs(a - b) for a, b in zip(r.y[row], fe)) <= 1e-12
        assert r.y[row, 0] == 0.0
    assert np.allclose(r.bound, np.cumsum(xf.astype(np.float64), axis=1), rtol=1e-14)


# ---------------------------------------------------------------- flags / indices

def pin_flag_compaction_and_indices(orc):
    g = load_golden("worked_example.txt")
    x = np.array(g["x"], np.int32)
    flags = np.array(g["flags"], np.uint8)
    out, c = orc.compact_flags(x, flags)
    assert out.tolist() == g["compacted"] and c == g["count"][0]
    idx, ci = orc.indices(flags=flags)
    # the kept positions, read off the page's flags by numpy, and their scan values
    assert idx.tolist() == np.flatnonzero(flags).tolist() and ci == c
    excl = orc.scan(flags.astype(np.int32), "sum", False).y
    assert excl[idx].tolist() == list(range(c))
    idx2, _ = orc.indices(x=x, cmp="gt", threshold=2)
    assert idx2.tolist() == idx.tolist()
    rng = np.random.default_rng(23)
    for n in (1, 10, 1000, 50_000):
        f = (rng.random(n) < 0.3).astype(np.uint8) * rng.integers(1, 256, n).astype(np.uint8)
        xv = rng.integers(-(1 << 31), 1 << 31, n, dtype=np.int64).astype(np.int32)
        out, c = orc.compact_flags(xv, f)
        assert np.array_equal(out, xv[f != 0]) and c == int(np.count_nonzero(f))
        assert np.array_equal(orc.indices(flags=f)[0], np.flatnonzero(f).astype(np.uint32))
        for cmp, fn in (("lt", np.less), ("ge", np.greater_equal), ("eq", np.equal)):
            want = np.flatnonzero(fn(xv, 17)).astype(np.uint32)
            assert np.array_equal(orc.indices(x=xv, cmp=cmp, threshold=17)[0], want)
        xf = xv.view(np.float32)
        out, c = orc.compact_flags(xf, f)
        assert _bits(out) == _bits(xf[f != 0])      # payload bits copied, whatever they are
    assert orc.indices(flags=np.zeros(0, np.uint8))[1] == 0


# ---------------------------------------------------------------- stable sort

def _order_key_np(dtype, bits_u32):
    """The sort order as unsigned integers, computed here with numpy bit operations
    (independent of the oracle): int32 flips the sign bit; float32 flips all bits of
    negatives and sets the sign bit of the rest (IEEE total order)."""
    b = bits_u32.astype(np.uint32)
    if dtype == "int32":
        return b ^ np.uint32(0x80000000)
    if dtype == "float32":
        neg = (b & np.uint32(0x80000000)) != 0
        return np.where(neg, ~b, b | np.uint32(0x80000000)).astype(np.uint32)
    return b


def pin_sort_matches_numpy_stable_argsort(orc):
    rng = np.random.default_rng(17)
    for dtype in ("int32", "uint32", "float32"):
        for n in (1, 2, 7, 100, 5000):
            if dtype == "float32":
                k = (rng.standard_normal(n) * 10).round().astype(np.float32)
                k[::5] = -0.0
            elif dtype == "int32":
                k = rng.integers(-50, 50, n).astype(np.int32)
            else:
                k = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
                k[::3] = 7
            v = np.arange(n, dtype=np.uint32)
            sk, sv = orc.sort(k, v)
            order = np.argsort(_order_key_np(dtype, k.view(np.uint32)), kind="stable")
            assert _bits(sk) == _bits(k[order])
            assert sv.tolist() == order.tolist()
            # keys only: the same keys
            assert _bits(orc.sort(k)[0]) == _bits(k[order])
    ints = rng.integers(-(1 << 31), 1 << 31, 3000, dtype=np.int64).astype(np.int32)
    assert np.array_equal(orc.sort(ints)[0], np.sort(ints))
    uints = ints.view(np.uint32)
    assert np.array_equal(orc.sort(uints)[0], np.sort(uints))


def pin_sort_brute_force_and_invariants(orc):
    rng = np.random.default_rng(19)
    for n in range(1, 9):
        for _ in range(20):
            k = rng.integers(-3, 3, n).astype(np.int32)
            v = np.arange(n, dtype=np.uint32)
            sk, sv = orc.sort(k, v)
            # insertion sort, stable by construction
            pairs = list(zip(k.tolist(), v.tolist()))
            for i in range(1, len(pairs)):
                j = i
                while j > 0 and pairs[j - 1][0] > pairs[j][0]:
                    pairs[j - 1], pairs[j] = pairs[j], pairs[j - 1]
                    j -= 1
            assert sk.tolist() == [p[0] for p in pairs]
            assert sv.tolist() == [p[1] for p in pairs]
    k = rng.integers(0, 20, 10000).astype(np.uint32)
    v = np.arange(10000, dtype=np.uint32)
    sk, sv = orc.sort(k, v)
    assert np.all(sk[1:] >= sk[:-1])                           # ordered
    assert np.array_equal(np.sort(sv), v)                       # a permutation
    assert np.array_equal(k[sv], sk)                            # values follow keys
    same = sk[1:] == sk[:-1]
    assert np.all(sv[1:][same] > sv[:-1][same])                 # stable
    f = np.array([np.nan, 1.0, -np.nan, -0.0, 0.0, -np.inf, np.inf, -1.0], np.float32)
    want = [-np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, np.inf, np.nan]
    assert _bits(orc.sort(f)[0]) == _bits(np.array(want, np.float32))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
