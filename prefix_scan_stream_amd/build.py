"""Build libscan.so for gfx950 in-tree with hipcc.

    python -m prefix_scan_stream_amd.build          # or build() from Python

Objects go to prefix_scan_stream_amd/_build/ (git-ignored); the shared library
to prefix_scan_stream_amd/libscan.so.  Only the entry points declared in
include/libscan.h are exported.

build_bounded_wait_test_lib() builds the same sources into libscan_spin1.so with
every bounded wait (look-back, chased prefixes) giving up after one empty poll.
Only the test of the workspace error word loads it; the package never does.
build_tiny_tile_lib() builds them into libscan_tiny.so with 256-element scan tiles,
for the tests that follow the pages' block decomposition tile by tile.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
HEADER = os.path.join(ROOT, "include", "libscan.h")
LIB = os.path.join(PKG, "libscan.so")
SPIN1_LIB = os.path.join(PKG, "libscan_spin1.so")
TINY_LIB = os.path.join(PKG, "libscan_tiny.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
          "-I", os.path.join(ROOT, "include")]
# Packed fp32 VALU forms are kept out of the generated code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = ["ls_scan.hip", "ls_compact.hip", "ls_batched.hip", "ls_sort.hip", "ls_segmented.hip",
           "ls_noalloc.hip", "ls_api.cpp"]


def exported_symbols() -> list[str]:
    """Function names declared in include/libscan.h."""
    with open(HEADER) as f:
        text = f.read()
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, re.M)
    return sorted(set(names))


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE, *defines, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *defines, f"--offload-arch={ARCH}", "-c", path, "-o", obj]
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = False, lib: str = LIB, build_dir: str = BUILD, defines: tuple = ()) -> str:
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    vs = os.path.join(build_dir, "exports.map")
    with open(vs, "w") as f:
        f.write("{\n  global:\n")
        for name in exported_symbols():
            f.write(f"    {name};\n")
        f.write("  local: *;\n};\n")
    tmp = lib + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
                           f"-Wl,--version-script={vs}"])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


CEILING_LIB = os.path.join(PKG, "libls_ceiling.so")
CEILING_HEADER = os.path.join(ROOT, "include", "ls_ceiling.h")


def build_ceiling_lib(verbose: bool = False) -> str:
    """libls_ceiling.so: the read / write / copy ceiling kernels the benchmark times
    beside the library (include/ls_ceiling.h); not part of libscan."""
    os.makedirs(BUILD, exist_ok=True)
    obj = _compile("ls_ceiling.hip")
    with open(CEILING_HEADER) as f:
        names = sorted(set(re.findall(r"^int\s+(ls_ceiling_[a-z]+)\s*\(", f.read(), re.M)))
    vs = os.path.join(BUILD, "ceiling_exports.map")
    with open(vs, "w") as f:
        f.write("{\n  global:\n" + "".join(f"    {n};\n" for n in names) + "  local: *;\n};\n")
    tmp = CEILING_LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj,
                           f"-Wl,--version-script={vs}"])
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print(f"built {CEILING_LIB}")
    return CEILING_LIB


def build_tiny_tile_lib(verbose: bool = False) -> str:
    """libscan_tiny.so: the scans with 256-element tiles (one wave, one run of four
    per thread), so that a handful of elements spans several tiles (test use only)."""
    return build(verbose, TINY_LIB, os.path.join(BUILD, "tiny"),
                 ("-DLS_SCAN_BLOCK=64", "-DLS_SCAN_CHUNKS=1", "-DLS_SP_BLOCK=64", "-DLS_SP_CHUNKS=1"))


def build_bounded_wait_test_lib(verbose: bool = False) -> str:
    """libscan_spin1.so: bounded waits give up after one empty poll (test use only)."""
    return build(verbose, SPIN1_LIB, os.path.join(BUILD, "spin1"), ("-DLS_WAIT_LIMIT_TICKS=0", "-DLS_FALLBACK_TICKS=0"))


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
