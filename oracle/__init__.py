"""CPU oracle for prefix scan and stream compaction (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  The product library never does, and this package imports nothing of
the product: it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain serial C, built with gcc); this
module only builds that file, marshals numpy arrays into it, and returns numpy
arrays.  ``brute.py`` holds a second, pure-Python O(n^2) definition used to pin
the C oracle on tiny inputs.

Codes (independent of the library header):
  dtype  "int32" | "uint32" | "float32"
  op     "sum" | "max" | "xor" | "min" | "and" | "or" | "prod" | "affine"
         (float32: sum, max, min, prod; affine: uint32 only)
  cmp    "lt" | "le" | "gt" | "ge" | "eq" | "ne"
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"int32": 0, "uint32": 1, "float32": 2}
OPS = {"sum": 0, "max": 1, "xor": 2, "min": 3, "and": 4, "or": 5, "prod": 6, "affine": 7}
CMPS = {"lt": 0, "le": 1, "gt": 2, "ge": 3, "eq": 4, "ne": 5}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (serial, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    U32 = ctypes.c_uint32
    lib.oracle_scan_u32.argtypes = [P, P, I64, I, I, I, P]
    lib.oracle_scan_u32.restype = I
    lib.oracle_scan_f32_sum.argtypes = [P, P, P, I64, I, P]
    lib.oracle_scan_f32_sum.restype = None
    lib.oracle_scan_f32_max.argtypes = [P, P, I64, I, P]
    lib.oracle_scan_f32_max.restype = None
    lib.oracle_scan_f32_min.argtypes = [P, P, I64, I, P]
    lib.oracle_scan_f32_min.restype = None
    lib.oracle_scan_f32_prod.argtypes = [P, P, I64, I, P]
    lib.oracle_scan_f32_prod.restype = None
    lib.oracle_batched_f32_min.argtypes = [P, P, I64, I64, I]
    lib.oracle_batched_f32_min.restype = None
    lib.oracle_batched_f32_prod.argtypes = [P, P, I64, I64, I]
    lib.oracle_batched_f32_prod.restype = None
    lib.oracle_compact.argtypes = [P, P, I64, I, I, U32]
    lib.oracle_compact.restype = I64
    lib.oracle_compact_via_scan.argtypes = [P, P, I64, I, I, U32, P, P]
    lib.oracle_compact_via_scan.restype = I64
    lib.oracle_batched_u32.argtypes = [P, P, I64, I64, I, I, I]
    lib.oracle_batched_u32.restype = I
    lib.oracle_batched_f32_sum.argtypes = [P, P, P, I64, I64, I]
    lib.oracle_batched_f32_sum.restype = None
    lib.oracle_batched_f32_max.argtypes = [P, P, I64, I64, I]
    lib.oracle_batched_f32_max.restype = None
    lib.oracle_segmented_u32.argtypes = [P, P, P, I64, I, I, I]
    lib.oracle_segmented_u32.restype = I
    lib.oracle_segmented_f32_sum.argtypes = [P, P, P, P, I64, I]
    lib.oracle_segmented_f32_sum.restype = None
    lib.oracle_segmented_f32_minmax.argtypes = [P, P, P, I64, I, I]
    lib.oracle_segmented_f32_minmax.restype = None
    lib.oracle_segmented_f32_prod.argtypes = [P, P, P, I64, I]
    lib.oracle_segmented_f32_prod.restype = None
    lib.oracle_heads_from_offsets.argtypes = [P, I64, P, I64]
    lib.oracle_heads_from_offsets.restype = I
    lib.oracle_stable_sort.argtypes = [P, P, I64, I, P, P]
    lib.oracle_stable_sort.restype = I
    lib.oracle_sort_order_key.argtypes = [I, U32]
    lib.oracle_sort_order_key.restype = U32
    lib.oracle_compact_flags.argtypes = [P, P, P, I64]
    lib.oracle_compact_flags.restype = I64
    lib.oracle_indices_flags.argtypes = [P, P, I64]
    lib.oracle_indices_flags.restype = I64
    lib.oracle_indices_if.argtypes = [P, P, I64, I, I, U32]
    lib.oracle_indices_if.restype = I64
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


def compile_variant(src_text: str, out_path: str) -> "Oracle":
    """Compile a modified copy of oracle.c (used by the tests that plant a mistake
    in the oracle and check that the pins catch it) and return an Oracle on it."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                           "-ffp-contract=off", "-o", out_path, c_path])
    return Oracle(_bind(ctypes.CDLL(out_path)))


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_name(x: np.ndarray) -> str:
    name = str(x.dtype)
    if name not in DTYPES:
        raise TypeError(f"oracle: unsupported dtype {x.dtype}")
    return name


class ScanResult:
    """y: the scan (int32/uint32/float32 arrays; float64 for a float32 sum);
    total: the value no exclusive cell holds (scalar of the same kind);
    bound: for a float32 sum, sum_{j<=i} |x_j| in float64, else None."""

    def __init__(self, y, total, bound=None):
        self.y = y
        self.total = total
        self.bound = bound


class Oracle:
    """The oracle routines bound to one compiled copy of oracle.c."""

    def __init__(self, lib):
        self._lib = lib

    def scan(self, x: np.ndarray, op: str = "sum", inclusive: bool = True) -> ScanResult:
        """Serial scan of a 1-D array (see oracle.c for the definitions)."""
        lib = self._lib
        x = np.ascontiguousarray(x)
        dt = _dtype_name(x)
        n = x.shape[0]
        inc = 1 if inclusive else 0
        if dt in ("int32", "uint32"):
            xu = x.view(np.uint32)
            y = np.empty(n, np.uint32)
            tot = np.zeros(1, np.uint32)
            rc = lib.oracle_scan_u32(_ptr(xu), _ptr(y), n, DTYPES[dt], OPS[op], inc, _ptr(tot))
            if rc:
                raise ValueError(f"oracle: bad op {op} for {dt}")
            return ScanResult(y.view(x.dtype), tot.view(x.dtype)[0])
        if op == "sum":
            y = np.empty(n, np.float64)
            b = np.empty(n, np.float64)
            tot = np.zeros(1, np.float64)
            lib.oracle_scan_f32_sum(_ptr(x), _ptr(y), _ptr(b), n, inc, _ptr(tot))
            return ScanResult(y, tot[0], b)
        if op in ("max", "min"):
            y = np.empty(n, np.float32)
            tot = np.zeros(1, np.float32)
            fn = lib.oracle_scan_f32_max if op == "max" else lib.oracle_scan_f32_min
            fn(_ptr(x), _ptr(y), n, inc, _ptr(tot))
            return ScanResult(y, tot[0])
        if op == "prod":
            y = np.empty(n, np.float64)
            tot = np.zeros(1, np.float64)
            lib.oracle_scan_f32_prod(_ptr(x), _ptr(y), n, inc, _ptr(tot))
            return ScanResult(y, tot[0])
        raise ValueError(f"oracle: op {op} is not defined for float32")

    def compact(self, x: np.ndarray, cmp: str, threshold, via_scan: bool = False):
        """Stable compaction: (kept elements in input order, count)."""
        lib = self._lib
        x = np.ascontiguousarray(x)
        dt = _dtype_name(x)
        thr = np.array([threshold], dtype=x.dtype).view(np.uint32)[0]
        n = x.shape[0]
        out = np.zeros(n + 1, np.uint32)  # one spare cell: never read back
        xu = x.view(np.uint32)
        if via_scan:
            flags = np.empty(max(n, 1), np.int64)
            index = np.empty(max(n, 1), np.int64)
            c = lib.oracle_compact_via_scan(_ptr(xu), _ptr(out), n, DTYPES[dt], CMPS[cmp],
                                            int(thr), _ptr(flags), _ptr(index))
        else:
            c = lib.oracle_compact(_ptr(xu), _ptr(out), n, DTYPES[dt], CMPS[cmp], int(thr))
        if c < 0:
            raise ValueError("oracle: bad compaction arguments")
        return out[:c].view(x.dtype).copy(), int(c)

    def batched(self, x: np.ndarray, op: str = "sum", inclusive: bool = False) -> ScanResult:
        """Row-wise scan of a 2-D row-major array; no carry between rows."""
        lib = self._lib
        x = np.ascontiguousarray(x)
        if x.ndim != 2:
            raise ValueError("oracle.batched wants a 2-D array")
        dt = _dtype_name(x)
        rows, cols = x.shape
        inc = 1 if inclusive else 0
        if dt in ("int32", "uint32"):
            y = np.empty((rows, cols), np.uint32)
            rc = lib.oracle_batched_u32(_ptr(x.view(np.uint32)), _ptr(y), rows, cols, DTYPES[dt],
                                        OPS[op], inc)
            if rc:
                raise ValueError(f"oracle: bad op {op} for {dt}")
            return ScanResult(y.view(x.dtype), None)
        if op == "sum":
            y = np.empty((rows, cols), np.float64)
            b = np.empty((rows, cols), np.float64)
            lib.oracle_batched_f32_sum(_ptr(x), _ptr(y), _ptr(b), rows, cols, inc)
            return ScanResult(y, None, b)
        if op in ("max", "min"):
            y = np.empty((rows, cols), np.float32)
            fn = lib.oracle_batched_f32_max if op == "max" else lib.oracle_batched_f32_min
            fn(_ptr(x), _ptr(y), rows, cols, inc)
            return ScanResult(y, None)
        if op == "prod":
            y = np.empty((rows, cols), np.float64)
            lib.oracle_batched_f32_prod(_ptr(x), _ptr(y), rows, cols, inc)
            return ScanResult(y, None)
        raise ValueError(f"oracle: op {op} is not defined for float32")


    def segmented(self, x: np.ndarray, op: str = "sum", inclusive: bool = True,
                  heads: np.ndarray | None = None, offsets: np.ndarray | None = None) -> ScanResult:
        """Segmented scan of a 1-D array; segments by head flags (bytes, nonzero =
        first element of a segment; element 0 always starts one) or by CSR offsets
        (int64, offsets[0] = 0 ... offsets[-1] = n)."""
        lib = self._lib
        x = np.ascontiguousarray(x)
        dt = _dtype_name(x)
        n = x.shape[0]
        if offsets is not None:
            off = np.ascontiguousarray(offsets, dtype=np.int64)
            h = np.zeros(max(n, 1), np.uint8)
            if lib.oracle_heads_from_offsets(_ptr(off), off.shape[0] - 1, _ptr(h), n):
                raise ValueError("oracle.segmented: offsets must run from 0 to n, non-decreasing")
        else:
            h = np.ascontiguousarray(heads, dtype=np.uint8)
            if h.shape[0] != n:
                raise ValueError("oracle.segmented: heads must have n bytes")
            if n == 0:
                h = np.zeros(1, np.uint8)
        inc = 1 if inclusive else 0
        if dt in ("int32", "uint32"):
            y = np.empty(n, np.uint32)
            if lib.oracle_segmented_u32(_ptr(x.view(np.uint32)), _ptr(y), _ptr(h), n, DTYPES[dt],
                                        OPS[op], inc):
                raise ValueError(f"oracle: bad op {op} for {dt}")
            return ScanResult(y.view(x.dtype), None)
        if op == "sum":
            y = np.empty(n, np.float64)
            b = np.empty(n, np.float64)
            lib.oracle_segmented_f32_sum(_ptr(x), _ptr(y), _ptr(b), _ptr(h), n, inc)
            return ScanResult(y, None, b)
        if op in ("max", "min"):
            y = np.empty(n, np.float32)
            lib.oracle_segmented_f32_minmax(_ptr(x), _ptr(y), _ptr(h), n, inc, 1 if op == "min" else 0)
            return ScanResult(y, None)
        if op == "prod":
            y = np.empty(n, np.float64)
            lib.oracle_segmented_f32_prod(_ptr(x), _ptr(y), _ptr(h), n, inc)
            return ScanResult(y, None)
        raise ValueError(f"oracle: op {op} is not defined for float32")

    def sort(self, keys: np.ndarray, values: np.ndarray | None = None):
        """Stable ascending sort of 32-bit keys in their type's order (float32: IEEE
        total order); values, when given, follow their keys.  Returns (keys, values)."""
        lib = self._lib
        k = np.ascontiguousarray(keys).copy()
        dt = _dtype_name(k)
        n = k.shape[0]
        ku = k.view(np.uint32)
        tk = np.empty(max(n, 1), np.uint32)
        v = None
        tv = None
        if values is not None:
            v = np.ascontiguousarray(values).copy()
            if v.dtype.itemsize != 4 or v.shape[0] != n:
                raise ValueError("oracle.sort: values must be n 32-bit elements")
            tv = np.empty(max(n, 1), np.uint32)
        rc = lib.oracle_stable_sort(_ptr(ku), None if v is None else _ptr(v.view(np.uint32)), n,
                                    DTYPES[dt], _ptr(tk), None if tv is None else _ptr(tv))
        if rc:
            raise ValueError("oracle.sort: bad dtype")
        return k, v

    def compact_flags(self, x: np.ndarray, flags: np.ndarray):
        """Elements of x (any 32-bit type) whose byte flag is nonzero, in order; count."""
        x = np.ascontiguousarray(x)
        f = np.ascontiguousarray(flags, dtype=np.uint8)
        n = x.shape[0]
        out = np.zeros(n + 1, np.uint32)
        c = self._lib.oracle_compact_flags(_ptr(x.view(np.uint32)), _ptr(f), _ptr(out), n)
        return out[:c].view(x.dtype).copy(), int(c)

    def indices(self, flags: np.ndarray = None, x: np.ndarray = None, cmp: str = None,
                threshold=None):
        """Positions i (uint32) with flags[i] != 0, or with (x[i] CMP threshold)."""
        out_n = (flags if flags is not None else x).shape[0]
        out = np.zeros(out_n + 1, np.uint32)
        if flags is not None:
            f = np.ascontiguousarray(flags, dtype=np.uint8)
            c = self._lib.oracle_indices_flags(_ptr(f), _ptr(out), out_n)
        else:
            x = np.ascontiguousarray(x)
            dt = _dtype_name(x)
            thr = np.array([threshold], dtype=x.dtype).view(np.uint32)[0]
            c = self._lib.oracle_indices_if(_ptr(x.view(np.uint32)), _ptr(out), out_n, DTYPES[dt],
                                            CMPS[cmp], int(thr))
        if c < 0:
            raise ValueError("oracle: bad index-selection arguments")
        return out[:c].copy(), int(c)

    def order_key(self, dtype: str, bits: int) -> int:
        return int(self._lib.oracle_sort_order_key(DTYPES[dtype], int(bits) & 0xFFFFFFFF))


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(_load())
    return _default


def scan(x: np.ndarray, op: str = "sum", inclusive: bool = True) -> ScanResult:
    return default().scan(x, op, inclusive)


def compact(x: np.ndarray, cmp: str, threshold, via_scan: bool = False):
    return default().compact(x, cmp, threshold, via_scan)


def batched(x: np.ndarray, op: str = "sum", inclusive: bool = False) -> ScanResult:
    return default().batched(x, op, inclusive)


def sort(keys: np.ndarray, values: np.ndarray | None = None):
    return default().sort(keys, values)


def compact_flags(x: np.ndarray, flags: np.ndarray):
    return default().compact_flags(x, flags)


def indices(flags=None, x=None, cmp=None, threshold=None):
    return default().indices(flags, x, cmp, threshold)


def segmented(x, op="sum", inclusive=True, heads=None, offsets=None):
    return default().segmented(x, op, inclusive, heads, offsets)


def fp32_sum_within_tolerance(got: np.ndarray, ref: ScanResult, rel: float = 1e-6,
                              abs_: float = 1e-6):
    """The float32 acceptance rule: |got_i - ref_i| <= rel * sum_{j<=i}|x_j| + abs.

    Returns (ok, worst_ratio, worst_index) where ratio = err / allowed."""
    got = np.asarray(got, np.float64).reshape(-1)
    y = np.asarray(ref.y, np.float64).reshape(-1)
    b = np.asarray(ref.bound, np.float64).reshape(-1)
    if got.size == 0:
        return True, 0.0, -1
    err = np.abs(got - y)
    allowed = rel * b + abs_
    ratio = err / allowed
    k = int(np.argmax(ratio))
    return bool(ratio[k] <= 1.0), float(ratio[k]), k
