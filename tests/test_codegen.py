"""Checks on the gfx950 code the kernels compile to (CPU only; hipcc cross-compiles).

Every kernel must keep its tile in registers: no private (scratch) segment and no
register spills -- a run-time index into a register array silently moves the tile
to per-lane scratch memory.  Packed fp32 VALU forms must not appear (the build
disables them)."""
import os
import re
import subprocess

import pytest

from prefix_scan_stream_amd import build as b

SOURCES = [s for s in b.SOURCES if s.endswith(".hip")]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in SOURCES:
        path = os.path.join(b.CSRC, src)
        s_file = os.path.join(d, src + ".s")
        subprocess.check_call([b.HIPCC, "-x", "hip", *b.COMMON, *b.DEVICE, "--cuda-device-only",
                               "-S", path, "-o", s_file], stderr=subprocess.DEVNULL)
        with open(s_file) as f:
            out[src] = f.read()
    return out


def kernel_metadata(text):
    """(name, private_segment_fixed_size, vgpr_spill_count) for each kernel."""
    names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
    priv = [int(v) for v in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", text, re.M)]
    spill = [int(v) for v in re.findall(r"^\s+\.vgpr_spill_count:\s+(\d+)", text, re.M)]
    return list(zip(names, priv, spill))


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_no_spills(asm, src):
    meta = kernel_metadata(asm[src])
    assert meta, f"no kernels found in {src}"
    for name, priv, spill in meta:
        assert priv == 0, f"{name} uses {priv} bytes of scratch"
        assert spill == 0, f"{name} spills {spill} VGPRs"


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32(asm, src):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm[src])


def test_status_words_use_device_coherent_accesses(asm):
    """The look-back's 64-bit status loads and stores carry the device-coherence bit."""
    text = asm["ls_scan.hip"]
    assert re.search(r"global_load_dwordx2 .* sc1", text)
    assert re.search(r"global_store_dwordx2 .* sc1", text)
