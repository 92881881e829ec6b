"""One status workspace serving scans, segmented scans and compactions in turn.

The words a call writes carry its epoch, and a call takes a word from an earlier
call as empty.  The three word formats keep the epoch's low bits at the same place,
so this holds across formats too: a compaction word written at epoch e must not read
as current to a scan or a segmented scan at a later epoch (it did, at epoch 16 e,
while the count word kept its epoch above the whole 36-bit count).

Each schedule starts from a freshly initialised workspace (epoch 0), puts a large
compaction at epoch 1, small scans after it (which rewrite only the first slot), and
a large scan or segmented scan at epoch 16, whose later tiles read slots last
written by that compaction; it then goes on mixing all three kinds.  Every result is
compared with a reference."""
import ctypes

import pytest
import torch

import prefix_scan_stream_amd as ps

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
INT32 = 0
SUM = 0
LT = 0
N = 1 << 22


def stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def test_mixed_calls_on_one_status_workspace():
    lib = ps.load_library()
    sizes = []
    for query, args in ((lib.ls_scan_workspace_bytes, (N, INT32, SUM)),
                        (lib.ls_compact_workspace_bytes, (N, INT32)),
                        (lib.ls_segmented_workspace_bytes, (N, INT32, SUM))):
        nb = ctypes.c_size_t(0)
        assert query(*args, ctypes.byref(nb)) == 0
        sizes.append(nb.value)
    ws = torch.empty(max(sizes), dtype=torch.uint8, device=DEV)
    assert lib.ls_workspace_init(ws.data_ptr(), ws.numel(), stream()) == 0

    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    big = torch.randint(0, 16, (N,), dtype=torch.int32, device=DEV, generator=g)
    small = big[:1000].clone()
    comp_in = torch.randint(0, 1 << 31, (N,), dtype=torch.int32, device=DEV, generator=g)
    heads = (torch.rand(N, device=DEV, generator=g) < 1.0 / 1024).to(torch.uint8)
    heads[0] = 1
    out = torch.empty_like(big)
    count = torch.empty(1, dtype=torch.int64, device=DEV)

    want_big = torch.cumsum(big.to(torch.int64), 0).to(torch.int32) - big
    want_small = torch.cumsum(small.to(torch.int64), 0).to(torch.int32) - small
    seg_id = torch.cumsum(heads.to(torch.int64), 0)
    csum = torch.cumsum(big.to(torch.int64), 0)
    starts = torch.nonzero(heads).flatten()
    base = torch.zeros(int(seg_id[-1]) + 1, dtype=torch.int64, device=DEV)
    base[1:] = csum[starts] - big[starts].to(torch.int64)
    want_seg = (csum - base[seg_id]).to(torch.int32)  # inclusive, restarting at every head

    ptr, nb, st = ws.data_ptr(), ws.numel(), stream()

    def compaction(epoch, thr):
        assert lib.compact_if(comp_in.data_ptr(), out.data_ptr(), count.data_ptr(), N, INT32, LT,
                              thr, ptr, nb, st) == 0
        want = comp_in[comp_in < thr]
        c = int(count.item())
        assert c == want.numel(), f"epoch {epoch}: count"
        assert torch.equal(out[:c], want), f"epoch {epoch}: compaction"

    def big_scan(epoch):
        assert lib.scan_exclusive(big.data_ptr(), out.data_ptr(), N, INT32, SUM, None, ptr, nb, st) == 0
        assert torch.equal(out, want_big), f"epoch {epoch}: scan"

    def segmented(epoch):
        assert lib.segmented_scan(big.data_ptr(), out.data_ptr(), N, INT32, SUM, 0, heads.data_ptr(),
                                  None, ptr, nb, st) == 0
        assert torch.equal(out, want_seg), f"epoch {epoch}: segmented scan"

    def small_scan(epoch):
        o = out[:1000]
        assert lib.scan_exclusive(small.data_ptr(), o.data_ptr(), 1000, INT32, SUM, None, ptr, nb, st) == 0
        assert torch.equal(o, want_small), f"epoch {epoch}: small scan"

    for at16 in (big_scan, segmented):
        print(f"schedule with {at16.__name__} at epoch 16", flush=True)
        assert lib.ls_workspace_init(ptr, nb, st) == 0
        schedule = {1: lambda e: compaction(e, 1 << 30), 16: at16, 17: lambda e: compaction(e, 1 << 29),
                    18: segmented, 19: big_scan, 20: lambda e: compaction(e, 1 << 28), 21: big_scan}
        for epoch in range(24):
            schedule.get(epoch, small_scan)(epoch)
    flags = ctypes.c_uint32(0)
    assert lib.ls_workspace_check(ptr, ctypes.byref(flags), st) == 0
    assert flags.value == 0
