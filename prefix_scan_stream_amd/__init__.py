"""prefix_scan_stream_amd -- Python binding of libscan (MI355X / gfx950).

A thin ctypes layer over the C ABI in include/libscan.h: it checks that tensors
live on a GPU, passes their pointers, sizes and the current HIP stream, and
raises LibscanError on a non-OK status.  Every step of the computation runs in
the library's HIP kernels; there is no other implementation behind these names,
and importing or calling them fails loudly when libscan.so is missing.

PyTorch supplies device memory and streams only.  Workspaces are cached per
(device, stream), zero-filled by the library once when they are made, and grown
on demand; a workspace that a larger one replaces is kept, not freed, because a
HIP graph captured earlier may still use it (release_workspaces() frees them).

Checked mode (set_checked(True), or LIBSCAN_CHECKED=1 in the environment) reads
the workspace's error word after every call that uses one -- which waits for the
stream -- and raises LibscanError(LS_ERR_INCOMPLETE) when a bounded wait inside
the call gave up, re-initialising the workspace.  It is off by default so that
calls stay asynchronous and can be captured in graphs.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

__all__ = [
    "LibscanError", "library_path", "load_library", "ls_abi_version", "ls_status_string",
    "ls_scan_workspace_bytes", "ls_compact_workspace_bytes", "scan_inclusive", "scan_exclusive",
    "compact_if", "batched_row_scan", "workspace_for", "scan_ex", "ls_scan_ex_workspace_bytes",
    "batched_row_scan_ex", "radix_sort", "ls_radix_sort_workspace_bytes", "compact_flags",
    "select_indices_if", "select_indices_flags",
    "segmented_scan", "ls_segmented_workspace_bytes", "scan_noalloc", "SCAN_NOALLOC_MAX_N",
    "ls_workspace_init", "ls_workspace_check", "set_checked", "workspace_error_flags",
    "release_workspaces",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libscan.so")

LS_OK, LS_ERR_INVALID_ARG, LS_ERR_UNSUPPORTED, LS_ERR_WORKSPACE, LS_ERR_HIP, LS_ERR_INCOMPLETE = range(6)
DTYPE_CODES = {"int32": 0, "uint32": 1, "float32": 2}
OP_CODES = {"sum": 0, "max": 1, "xor": 2, "min": 3, "and": 4, "or": 5, "prod": 6, "affine": 7}
CMP_CODES = {"lt": 0, "le": 1, "gt": 2, "ge": 3, "eq": 4, "ne": 5}
SCHEME_CODES = {"single_pass": 0, "reduce_then_scan": 1, "scan_then_propagate": 2,
                "deterministic": 3}
BLOCK_SCAN_CODES = {"wave_dpp": 0, "hillis_steele": 1, "hillis_steele_double": 2, "blelloch": 3}
_TORCH_DTYPES = {torch.int32: "int32", torch.float32: "float32"}
if hasattr(torch, "uint32"):
    _TORCH_DTYPES[torch.uint32] = "uint32"

SCAN_NOALLOC_MAX_N = 402653184  # LS_SCAN_NOALLOC_MAX_N

_lock = threading.Lock()
_lib = None
ABI_VERSION = 5  # the libscan.h version this binding marshals for
_checked = os.environ.get("LIBSCAN_CHECKED", "0") not in ("", "0")


class LibscanError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = ls_status_string(status) if _lib is not None else f"status {status}"
        super().__init__(f"{where}: {msg}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libscan.so (built in-tree by prefix_scan_stream_amd.build)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"libscan.so not found at {_LIB_PATH}; build it with "
                "`python -m prefix_scan_stream_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I, U32, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                              ctypes.c_size_t)
        lib.ls_abi_version.argtypes = []
        lib.ls_abi_version.restype = I
        if lib.ls_abi_version() != ABI_VERSION:
            raise ImportError(f"{_LIB_PATH} has ABI version {lib.ls_abi_version()}, this binding "
                              f"needs {ABI_VERSION}; rebuild with `python -m prefix_scan_stream_amd.build`")
        lib.ls_status_string.argtypes = [I]
        lib.ls_status_string.restype = ctypes.c_char_p
        lib.ls_workspace_init.argtypes = [P, SZ, P]
        lib.ls_workspace_init.restype = I
        lib.ls_workspace_check.argtypes = [P, ctypes.POINTER(U32), P]
        lib.ls_workspace_check.restype = I
        lib.ls_scan_workspace_bytes.argtypes = [I64, I, I, ctypes.POINTER(SZ)]
        lib.ls_scan_workspace_bytes.restype = I
        lib.ls_compact_workspace_bytes.argtypes = [I64, I, ctypes.POINTER(SZ)]
        lib.ls_compact_workspace_bytes.restype = I
        for name in ("scan_inclusive", "scan_exclusive"):
            fn = getattr(lib, name)
            fn.argtypes = [P, P, I64, I, I, P, P, SZ, P]
            fn.restype = I
        lib.ls_scan_ex_workspace_bytes.argtypes = [I64, I, I, I, ctypes.POINTER(SZ)]
        lib.ls_scan_ex_workspace_bytes.restype = I
        lib.scan_ex.argtypes = [P, P, I64, I, I, I, I, P, P, SZ, P]
        lib.ls_segmented_workspace_bytes.argtypes = [I64, I, I, ctypes.POINTER(SZ)]
        lib.ls_segmented_workspace_bytes.restype = I
        lib.segmented_scan.argtypes = [P, P, I64, I, I, I, P, P, P, SZ, P]
        lib.segmented_scan.restype = I
        lib.segmented_scan_offsets.argtypes = [P, P, I64, I, I, I, P, I64, P, P, SZ, P]
        lib.segmented_scan_offsets.restype = I
        lib.scan_ex.restype = I
        lib.batched_row_scan_ex.argtypes = [P, P, I64, I64, I, I, I, I, P]
        lib.batched_row_scan_ex.restype = I
        lib.compact_flags.argtypes = [P, P, P, P, I64, P, SZ, P]
        lib.compact_flags.restype = I
        lib.select_indices_if.argtypes = [P, P, P, I64, I, I, U32, P, SZ, P]
        lib.select_indices_if.restype = I
        lib.select_indices_flags.argtypes = [P, P, P, I64, P, SZ, P]
        lib.select_indices_flags.restype = I
        lib.ls_radix_sort_workspace_bytes.argtypes = [I64, I, I, ctypes.POINTER(SZ)]
        lib.ls_radix_sort_workspace_bytes.restype = I
        lib.radix_sort.argtypes = [P, P, P, P, I64, I, P, SZ, P]
        lib.radix_sort.restype = I
        lib.scan_noalloc.argtypes = [P, P, I64, I, I, I, P, P]
        lib.scan_noalloc.restype = I
        lib.compact_if.argtypes = [P, P, P, I64, I, I, U32, P, SZ, P]
        lib.compact_if.restype = I
        lib.batched_row_scan.argtypes = [P, P, I64, I64, I, I, I, P]
        lib.batched_row_scan.restype = I
        _lib = lib
        return lib


def ls_abi_version() -> int:
    return load_library().ls_abi_version()


def ls_status_string(status: int) -> str:
    return load_library().ls_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != LS_OK:
        raise LibscanError(status, where)


def ls_scan_workspace_bytes(n: int, dtype: str, op: str) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ls_scan_workspace_bytes(n, DTYPE_CODES[dtype], OP_CODES[op],
                                                  ctypes.byref(out)), "ls_scan_workspace_bytes")
    return out.value


def ls_scan_ex_workspace_bytes(n: int, dtype: str, op: str, scheme: str) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ls_scan_ex_workspace_bytes(n, DTYPE_CODES[dtype], OP_CODES[op],
                                                     SCHEME_CODES[scheme], ctypes.byref(out)),
           "ls_scan_ex_workspace_bytes")
    return out.value


def ls_compact_workspace_bytes(n: int, dtype: str) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ls_compact_workspace_bytes(n, DTYPE_CODES[dtype], ctypes.byref(out)),
           "ls_compact_workspace_bytes")
    return out.value


# ------------------------------------------------------------ workspaces

_ws_cache: dict = {}    # (device index, stream handle) -> the uint8 workspace in use
_ws_uses: dict = {}     # calls on each cached status workspace since its last initialisation
STATUS_REINIT_CALLS = 1 << 25
_ws_retired: list = []  # workspaces replaced by larger ones, kept for graphs that captured them


def set_checked(on: bool = True) -> None:
    """Checked mode: after each call that uses a workspace, wait for the stream and
    raise LibscanError(LS_ERR_INCOMPLETE) if a bounded wait in the call gave up."""
    global _checked
    _checked = bool(on)


def ls_workspace_init(ws: torch.Tensor, stream=None) -> None:
    """Zero-fill a uint8 device workspace (before first use) on `stream` (default:
    the current stream)."""
    _require_gpu(ws)
    s = stream if stream is not None else torch.cuda.current_stream(ws.device)
    _check(load_library().ls_workspace_init(_ptr(ws), ws.numel(), ctypes.c_void_p(s.cuda_stream)),
           "ls_workspace_init")


def ls_workspace_check(ws: torch.Tensor, stream=None) -> int:
    """The workspace's error bits (0: no call on it gave up a wait since it was last
    initialised).  Waits for `stream` (default: the current stream)."""
    _require_gpu(ws)
    s = stream if stream is not None else torch.cuda.current_stream(ws.device)
    flags = ctypes.c_uint32(0)
    st = load_library().ls_workspace_check(_ptr(ws), ctypes.byref(flags), ctypes.c_void_p(s.cuda_stream))
    if st not in (LS_OK, LS_ERR_INCOMPLETE):
        _check(st, "ls_workspace_check")
    return flags.value


def workspace_for(device: torch.device, stream: torch.cuda.Stream, nbytes: int,
                  kind: str = "status") -> torch.Tensor:
    """The cached, initialised uint8 workspace of (device, stream, kind), of at least
    nbytes.  Kinds keep apart what the C ABI requires to be apart: "status" for the
    single-pass scans, segmented scans and compactions (tile status words that must
    never be overwritten with other data), "sort" for the radix sort and "phases"
    for the three-phase scan_ex schemes (plain scratch)."""
    key = (device.index, stream.cuda_stream, kind)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        size = (max(nbytes, 1 << 16) + 255) & ~255
        new = torch.empty(size, dtype=torch.uint8, device=device)
        ls_workspace_init(new, stream)
        if buf is not None:
            _ws_retired.append(buf)
        _ws_cache[key] = new
        _ws_uses[key] = 0
        buf = new
    elif kind == "status":
        # status words compare epochs modulo 2^26: zero the workspace again well
        # before that many calls (one fill kernel per 2^25 calls)
        _ws_uses[key] = _ws_uses.get(key, 0) + 1
        if _ws_uses[key] >= STATUS_REINIT_CALLS:
            ls_workspace_init(buf, stream)
            _ws_uses[key] = 0
    return buf


def workspace_error_flags(device=None, stream=None) -> int:
    """Error bits of the cached workspace of (device, stream) (defaults: cuda:0's
    current stream); 0 when there is none yet.  Waits for the stream."""
    device = torch.device(device if device is not None else "cuda:0")
    s = stream if stream is not None else torch.cuda.current_stream(device)
    buf = _ws_cache.get((device.index, s.cuda_stream, "status"))
    return 0 if buf is None else ls_workspace_check(buf, s)


def release_workspaces() -> None:
    """Drop every cached and retired workspace (no graph that used one may be
    replayed afterwards)."""
    _ws_cache.clear()
    _ws_retired.clear()
    _ws_uses.clear()


def _after_call(ws: torch.Tensor, stream, where: str) -> None:
    """Checked mode: report a call whose bounded wait gave up."""
    if not _checked:
        return
    flags = ls_workspace_check(ws, stream)
    if flags:
        ls_workspace_init(ws, stream)
        raise LibscanError(LS_ERR_INCOMPLETE, f"{where} (workspace error bits {flags:#x})")


def _dtype_of(x: torch.Tensor) -> str:
    try:
        return _TORCH_DTYPES[x.dtype]
    except KeyError:
        raise TypeError(f"libscan: unsupported dtype {x.dtype} (int32, uint32, float32)") from None


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libscan: tensors must be on a GPU device")


def _stream_handle(device) -> tuple:
    s = torch.cuda.current_stream(device)
    return s, ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------ entry points

def _scan(name: str, x: torch.Tensor, op: str, out, total):
    lib = load_library()
    _require_gpu(x, out, total)
    if not x.is_contiguous():
        raise ValueError("libscan: input must be contiguous")
    dt = _dtype_of(x)
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != x.numel() or not out.is_contiguous():
        raise ValueError("libscan: out must be a contiguous tensor like the input")
    if total is not None and (total.dtype != x.dtype or total.numel() < 1):
        raise ValueError("libscan: total must hold one element of the input dtype")
    n = x.numel()
    stream, sh = _stream_handle(x.device)
    need = ls_scan_workspace_bytes(n, dt, op)
    ws = workspace_for(x.device, stream, need)
    st = getattr(lib, name)(_ptr(x), _ptr(out), n, DTYPE_CODES[dt], OP_CODES[op], _ptr(total),
                            _ptr(ws), ws.numel(), sh)
    _check(st, name)
    _after_call(ws, stream, name)
    return out


def ls_segmented_workspace_bytes(n: int, dtype: str = "int32", op: str = "sum") -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ls_segmented_workspace_bytes(n, DTYPE_CODES[dtype], OP_CODES[op],
                                                       ctypes.byref(out)), "ls_segmented_workspace_bytes")
    return out.value


def segmented_scan(x: torch.Tensor, op: str = "sum", exclusive: bool = False,
                   heads: torch.Tensor | None = None, offsets: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, total: torch.Tensor | None = None) -> torch.Tensor:
    """Scan each segment of the flattened x on its own.  Segments by `heads` (n bytes,
    nonzero = first element of a segment; element 0 always starts one) or by
    `offsets` (int64 CSR offsets, nseg + 1 entries from 0 to n); exactly one of the
    two.  total (optional, one element): the inclusive value of the last element."""
    lib = load_library()
    _require_gpu(x, heads, offsets, out, total)
    if (heads is None) == (offsets is None):
        raise ValueError("libscan: give exactly one of heads and offsets")
    if not x.is_contiguous():
        raise ValueError("libscan: input must be contiguous")
    dt = _dtype_of(x)
    n = x.numel()
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != n or not out.is_contiguous():
        raise ValueError("libscan: out must be a contiguous tensor like the input")
    if total is not None and (total.dtype != x.dtype or total.numel() < 1):
        raise ValueError("libscan: total must hold one element of the input dtype")
    stream, sh = _stream_handle(x.device)
    ws = workspace_for(x.device, stream, ls_segmented_workspace_bytes(n, dt, op))
    excl = 1 if exclusive else 0
    if heads is not None:
        heads = _flags_tensor(heads, n)
        st = lib.segmented_scan(_ptr(x), _ptr(out), n, DTYPE_CODES[dt], OP_CODES[op], excl, _ptr(heads),
                                _ptr(total), _ptr(ws), ws.numel(), sh)
        _check(st, "segmented_scan")
        _after_call(ws, stream, "segmented_scan")
    else:
        if offsets.dtype != torch.int64 or not offsets.is_contiguous() or offsets.numel() < 1:
            raise ValueError("libscan: offsets must be a contiguous int64 tensor of nseg + 1 entries")
        st = lib.segmented_scan_offsets(_ptr(x), _ptr(out), n, DTYPE_CODES[dt], OP_CODES[op], excl,
                                        _ptr(offsets), offsets.numel() - 1, _ptr(total), _ptr(ws),
                                        ws.numel(), sh)
        _check(st, "segmented_scan_offsets")
        _after_call(ws, stream, "segmented_scan_offsets")
    return out


def scan_inclusive(x: torch.Tensor, op: str = "sum", out: torch.Tensor | None = None,
                   total: torch.Tensor | None = None) -> torch.Tensor:
    """out[i] = x[0] (+) ... (+) x[i] over the flattened tensor; total (optional,
    one element) receives the reduction of all of x.  out may be x (in place)."""
    return _scan("scan_inclusive", x, op, out, total)


def scan_exclusive(x: torch.Tensor, op: str = "sum", out: torch.Tensor | None = None,
                   total: torch.Tensor | None = None) -> torch.Tensor:
    """out[0] = identity, out[i] = x[0] (+) ... (+) x[i-1]."""
    return _scan("scan_exclusive", x, op, out, total)


def scan_noalloc(x: torch.Tensor, op: str = "sum", exclusive: bool = False,
                 out: torch.Tensor | None = None, total: torch.Tensor | None = None) -> torch.Tensor:
    """The scan on the library's fixed per-GPU workspace (no workspace argument, no
    allocation inside the call; n <= LS_SCAN_NOALLOC_MAX_N).  Calls that may overlap
    on one GPU race: keep them on one stream.  With out and total given, this
    function allocates nothing either."""
    lib = load_library()
    _require_gpu(x, out, total)
    if not x.is_contiguous():
        raise ValueError("libscan: input must be contiguous")
    dt = _dtype_of(x)
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != x.numel() or not out.is_contiguous():
        raise ValueError("libscan: out must be a contiguous tensor like the input")
    if total is not None and (total.dtype != x.dtype or total.numel() < 1):
        raise ValueError("libscan: total must hold one element of the input dtype")
    _, sh = _stream_handle(x.device)
    st = lib.scan_noalloc(_ptr(x), _ptr(out), x.numel(), DTYPE_CODES[dt], OP_CODES[op],
                          1 if exclusive else 0, _ptr(total), sh)
    _check(st, "scan_noalloc")
    return out


def scan_ex(x: torch.Tensor, op: str = "sum", inclusive: bool = True,
            scheme: str = "single_pass", out: torch.Tensor | None = None,
            total: torch.Tensor | None = None) -> torch.Tensor:
    """A scan with an explicit device-wide scheme: "single_pass",
    "reduce_then_scan" or "scan_then_propagate" (see ls_scheme in libscan.h)."""
    lib = load_library()
    _require_gpu(x, out, total)
    if not x.is_contiguous():
        raise ValueError("libscan: input must be contiguous")
    dt = _dtype_of(x)
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != x.numel() or not out.is_contiguous():
        raise ValueError("libscan: out must be a contiguous tensor like the input")
    if total is not None and (total.dtype != x.dtype or total.numel() < 1):
        raise ValueError("libscan: total must hold one element of the input dtype")
    n = x.numel()
    stream, sh = _stream_handle(x.device)
    need = ls_scan_ex_workspace_bytes(n, dt, op, scheme)
    phases = scheme in ("reduce_then_scan", "scan_then_propagate")
    ws = workspace_for(x.device, stream, need, "phases" if phases else "status")
    st = lib.scan_ex(_ptr(x), _ptr(out), n, DTYPE_CODES[dt], OP_CODES[op], 0 if inclusive else 1,
                     SCHEME_CODES[scheme], _ptr(total), _ptr(ws), ws.numel(), sh)
    _check(st, "scan_ex")
    if not phases:  # the three-phase schemes never wait, and keep no error word
        _after_call(ws, stream, "scan_ex")
    return out


def compact_if(x: torch.Tensor, cmp: str, threshold, out: torch.Tensor | None = None,
               count: torch.Tensor | None = None):
    """Stable compaction of the flattened x under (x CMP threshold).

    Returns (out, count): out has x's size, its first `count` cells hold the kept
    elements in input order; count is a one-element int64 device tensor."""
    lib = load_library()
    _require_gpu(x, out, count)
    if not x.is_contiguous():
        raise ValueError("libscan: input must be contiguous")
    dt = _dtype_of(x)
    if out is None:
        out = torch.empty_like(x)
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=x.device)
    if count.dtype != torch.int64:
        raise ValueError("libscan: count must be int64")
    thr_bits = _threshold_bits(dt, threshold)
    n = x.numel()
    stream, sh = _stream_handle(x.device)
    need = ls_compact_workspace_bytes(n, dt)
    ws = workspace_for(x.device, stream, need)
    st = lib.compact_if(_ptr(x), _ptr(out), _ptr(count), n, DTYPE_CODES[dt], CMP_CODES[cmp],
                        thr_bits, _ptr(ws), ws.numel(), sh)
    _check(st, "compact_if")
    _after_call(ws, stream, "compact_if")
    return out, count


def _threshold_bits(dt: str, threshold) -> int:
    np_dt = {"int32": "i4", "uint32": "u4", "float32": "f4"}[dt]
    return int(np.array([threshold], dtype=np_dt).view(np.uint32)[0])


def _count_tensor(count, device):
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=device)
    if count.dtype != torch.int64:
        raise ValueError("libscan: count must be int64")
    return count


def _flags_tensor(flags: torch.Tensor, n: int) -> torch.Tensor:
    if flags.dtype not in (torch.uint8, torch.bool, torch.int8) or flags.numel() != n:
        raise ValueError("libscan: flags must be n bytes (uint8 / bool)")
    if not flags.is_contiguous():
        raise ValueError("libscan: flags must be contiguous")
    return flags


def compact_flags(x: torch.Tensor, flags: torch.Tensor, out: torch.Tensor | None = None,
                  count: torch.Tensor | None = None):
    """Stable compaction of the 32-bit elements of x whose byte flag is nonzero.
    Returns (out, count) like compact_if."""
    lib = load_library()
    _require_gpu(x, flags, out, count)
    if not x.is_contiguous() or x.element_size() != 4:
        raise ValueError("libscan: x must be a contiguous tensor of 32-bit elements")
    n = x.numel()
    flags = _flags_tensor(flags, n)
    if out is None:
        out = torch.empty_like(x)
    count = _count_tensor(count, x.device)
    stream, sh = _stream_handle(x.device)
    ws = workspace_for(x.device, stream, ls_compact_workspace_bytes(n, "uint32"))
    st = lib.compact_flags(_ptr(x), _ptr(flags), _ptr(out), _ptr(count), n, _ptr(ws), ws.numel(), sh)
    _check(st, "compact_flags")
    _after_call(ws, stream, "compact_flags")
    return out, count


def select_indices_if(x: torch.Tensor, cmp: str, threshold, out: torch.Tensor | None = None,
                      count: torch.Tensor | None = None):
    """Positions (int32 tensor holding uint32 values) of the elements with
    (x CMP threshold), ascending; returns (indices, count)."""
    lib = load_library()
    _require_gpu(x, out, count)
    if not x.is_contiguous():
        raise ValueError("libscan: input must be contiguous")
    dt = _dtype_of(x)
    n = x.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=x.device)
    count = _count_tensor(count, x.device)
    stream, sh = _stream_handle(x.device)
    ws = workspace_for(x.device, stream, ls_compact_workspace_bytes(n, dt))
    st = lib.select_indices_if(_ptr(x), _ptr(out), _ptr(count), n, DTYPE_CODES[dt], CMP_CODES[cmp],
                               _threshold_bits(dt, threshold), _ptr(ws), ws.numel(), sh)
    _check(st, "select_indices_if")
    _after_call(ws, stream, "select_indices_if")
    return out, count


def select_indices_flags(flags: torch.Tensor, out: torch.Tensor | None = None,
                         count: torch.Tensor | None = None):
    """Positions (int32 tensor holding uint32 values) of the nonzero flag bytes."""
    lib = load_library()
    _require_gpu(flags, out, count)
    n = flags.numel()
    flags = _flags_tensor(flags, n)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=flags.device)
    count = _count_tensor(count, flags.device)
    stream, sh = _stream_handle(flags.device)
    ws = workspace_for(flags.device, stream, ls_compact_workspace_bytes(n, "uint32"))
    st = lib.select_indices_flags(_ptr(flags), _ptr(out), _ptr(count), n, _ptr(ws), ws.numel(), sh)
    _check(st, "select_indices_flags")
    _after_call(ws, stream, "select_indices_flags")
    return out, count


def batched_row_scan(x: torch.Tensor, op: str = "sum", exclusive: bool = True,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Scan each row of a contiguous 2-D tensor independently (no carry between rows)."""
    lib = load_library()
    _require_gpu(x, out)
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("libscan: batched_row_scan wants a contiguous 2-D tensor")
    dt = _dtype_of(x)
    if out is None:
        out = torch.empty_like(x)
    rows, cols = x.shape
    _, sh = _stream_handle(x.device)
    st = lib.batched_row_scan(_ptr(x), _ptr(out), rows, cols, DTYPE_CODES[dt], OP_CODES[op],
                              1 if exclusive else 0, sh)
    _check(st, "batched_row_scan")
    return out


def batched_row_scan_ex(x: torch.Tensor, op: str = "sum", exclusive: bool = True,
                        block_scan: str = "wave_dpp", out: torch.Tensor | None = None) -> torch.Tensor:
    """batched_row_scan with an explicit block-level scan: "wave_dpp",
    "hillis_steele", "hillis_steele_double" or "blelloch" (see ls_block_scan)."""
    lib = load_library()
    _require_gpu(x, out)
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("libscan: batched_row_scan wants a contiguous 2-D tensor")
    dt = _dtype_of(x)
    if out is None:
        out = torch.empty_like(x)
    rows, cols = x.shape
    _, sh = _stream_handle(x.device)
    st = lib.batched_row_scan_ex(_ptr(x), _ptr(out), rows, cols, DTYPE_CODES[dt], OP_CODES[op],
                                 1 if exclusive else 0, BLOCK_SCAN_CODES[block_scan], sh)
    _check(st, "batched_row_scan_ex")
    return out


def ls_radix_sort_workspace_bytes(n: int, dtype: str, with_values: bool) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ls_radix_sort_workspace_bytes(n, DTYPE_CODES[dtype], 1 if with_values else 0,
                                                        ctypes.byref(out)),
           "ls_radix_sort_workspace_bytes")
    return out.value


def radix_sort(keys: torch.Tensor, values: torch.Tensor | None = None,
               out_keys: torch.Tensor | None = None, out_values: torch.Tensor | None = None):
    """Stable ascending sort of a flat 32-bit key tensor (int32 / uint32 / float32 in
    IEEE total order), with optional 32-bit values.  Returns (keys, values or None)."""
    lib = load_library()
    _require_gpu(keys, values, out_keys, out_values)
    if not keys.is_contiguous() or (values is not None and not values.is_contiguous()):
        raise ValueError("libscan: keys and values must be contiguous")
    dt = _dtype_of(keys)
    n = keys.numel()
    if values is not None and (values.numel() != n or values.element_size() != 4):
        raise ValueError("libscan: values must hold n 32-bit elements")
    if out_keys is None:
        out_keys = torch.empty_like(keys)
    if values is not None and out_values is None:
        out_values = torch.empty_like(values)
    stream, sh = _stream_handle(keys.device)
    need = ls_radix_sort_workspace_bytes(n, dt, values is not None)
    ws = workspace_for(keys.device, stream, need, "sort")
    st = lib.radix_sort(_ptr(keys), _ptr(out_keys), _ptr(values), _ptr(out_values), n, DTYPE_CODES[dt],
                        _ptr(ws), ws.numel(), sh)
    _check(st, "radix_sort")
    _after_call(ws, stream, "radix_sort")
    return out_keys, (out_values if values is not None else None)

