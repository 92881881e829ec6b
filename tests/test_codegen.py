"""Checks on the gfx950 code the kernels compile to (CPU only; hipcc cross-compiles).

Every kernel must keep its tile in registers: no private (scratch) segment and no
register spills -- a run-time index into a register array silently moves the tile
to per-lane scratch memory.  Packed fp32 VALU forms must not appear (the compile
flags disable them)."""
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


def kernel_body(text, mangled_prefix):
    """Assembly of the first kernel whose symbol starts with mangled_prefix."""
    lines = text.split("\n")
    for i, line in enumerate(lines):
        if line.startswith(mangled_prefix) and line.split(";")[0].rstrip().endswith(":"):
            body = []
            for l2 in lines[i + 1:]:
                body.append(l2)
                if "s_endpgm" in l2:
                    return "\n".join(body)
    raise AssertionError(f"kernel {mangled_prefix} not found")


@pytest.mark.parametrize("src,prefix,runs", [
    ("ls_scan.hip", "_ZN2ls23scan_single_pass_kernelINS_6SumU32ELb0ELb1ELi14ELb0E", 14),
    ("ls_scan.hip", "_ZN2ls23scan_single_pass_kernelINS_6SumF32ELb0ELb1ELi16ELb1E", 16),
    ("ls_scan.hip", "_ZN2ls18tile_reduce_kernelINS_6SumU32ELb1E", 16),
    ("ls_scan.hip", "_ZN2ls16tile_scan_kernelINS_6SumU32ELb0ELb1E", 16),
    ("ls_scan.hip", "_ZN2ls17add_offset_kernelINS_6SumU32ELb1E", 16),
    ("ls_compact.hip", "_ZN2ls14compact_kernelILi0ELb1E", 8),
])
def test_aligned_tiles_load_128_bits(asm, src, prefix, runs):
    """Aligned tiles are read with 128-bit loads only (one per run of 4 elements; the
    single pass has 14 runs per thread, its deterministic form 16)."""
    body = kernel_body(asm[src], prefix)
    assert len(re.findall(r"buffer_load_dwordx4", body)) >= runs
    assert not re.search(r"buffer_load_dword\s", body)


def _vregs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


@pytest.mark.parametrize("src", SOURCES)
def test_wide_stores_keep_their_data_wait_state(asm, src):
    """A store of more than 64 bits reads its data registers after it issues; a VALU
    write to them right behind it needs one wait state.  The compiler inserts it
    only when a buffer store's soffset is not a register, so no 96/128-bit buffer
    store may take a register soffset, and no VALU may overwrite a wide store's data
    as the very next instruction (that race stored wrong values on gfx950)."""
    text = asm[src]
    assert not re.search(r"buffer_store_dwordx[34] v\[\d+:\d+\], v\d+, s\[\d+:\d+\], s\d+", text)
    ins = [l.strip() for l in text.split("\n")]
    ins = [l for l in ins if l and not l.startswith((".", ";")) and not l.endswith(":")]
    for k, line in enumerate(ins[:-1]):
        m = re.match(r"(buffer|global)_store_dwordx[34]\s", line)
        if not m:
            continue
        ops = [p.strip() for p in line.split(None, 1)[1].split(",")]
        data = _vregs(ops[1] if m.group(1) == "global" else ops[0])
        nxt = ins[k + 1]
        if nxt.startswith("v_"):
            dst = nxt.split(None, 1)[1].split(",")[0].strip()
            assert not (_vregs(dst) & data), f"{src}: '{line}' then '{nxt}'"


@pytest.mark.parametrize("src", [s for s in SOURCES if s != "ls_ceiling.hip"])
def test_no_cache_writeback_or_invalidate(asm, src):
    """Tile hand-off uses relaxed device-coherent loads and stores only.  A release
    or acquire at device scope would add an L2 writeback (buffer_wbl2) or invalidate
    (buffer_inv); one per block once made the 2^28 scan 2.5 times slower."""
    assert not re.search(r"\bbuffer_(wbl2|inv)\b", asm[src])
