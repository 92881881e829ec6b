"""The library's calls can be captured in a HIP graph and replayed.

A call launches only kernels (a workspace is zero-filled by a kernel, not a memset),
so torch.cuda.graph can capture it.  The graph is replayed several times with eager
work by the library in between (other inputs, the same entry points), and every
replay is compared element by element with the result of an eager call."""
import numpy as np
import pytest
import torch

import prefix_scan_stream_amd as ps
import workloads as wl
from gpu_util import DEV, bits, to_dev, to_host

pytestmark = pytest.mark.gpu

N = 40 * 28672 + 11      # the scan: 41 tiles, the last one ragged
NC = 18 * 16384 + 5       # compaction: 19 tiles, the last one ragged


def test_replays_match_eager_calls():
    x = to_dev(wl.int_uniform(N, 0, 16, seed=950))
    xc = to_dev(wl.int_uniform(NC, -1000, 1000, seed=951))
    rows = to_dev(wl.rows64(4096))
    thr = 0

    y_ref = to_host(ps.scan_exclusive(x, "sum"))
    o_ref, c_ref = ps.compact_if(xc, "lt", thr)
    c_ref = int(to_host(c_ref)[0])
    o_ref = to_host(o_ref)[:c_ref]
    r_ref = to_host(ps.batched_row_scan(rows, "sum", True))

    y = torch.empty_like(x)
    o = torch.empty_like(xc)
    cnt = torch.empty(1, dtype=torch.int64, device=DEV)
    r = torch.empty_like(rows)

    def work():
        ps.scan_exclusive(x, "sum", out=y)
        ps.compact_if(xc, "lt", thr, out=o, count=cnt)
        ps.batched_row_scan(rows, "sum", True, out=r)

    # warm up on a side stream (the binding's per-stream workspace is made there)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()

    other = to_dev(wl.int_uniform(N, 0, 16, seed=952))
    for rep in range(4):
        y.fill_(-7)
        o.fill_(-7)
        cnt.fill_(-7)
        r.fill_(-7.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(y)), bits(y_ref)), f"replay {rep}: scan"
        c = int(to_host(cnt)[0])
        assert c == c_ref, f"replay {rep}: count {c} != {c_ref}"
        assert np.array_equal(to_host(o)[:c], o_ref), f"replay {rep}: compaction"
        assert np.array_equal(bits(to_host(r)), bits(r_ref)), f"replay {rep}: batched rows"
        # eager calls between replays, on other data
        ps.scan_exclusive(other, "sum")
        ps.compact_if(other, "lt", 8)
        torch.cuda.synchronize()


def test_earlier_graph_survives_a_larger_capture():
    """Two captures on the same (default capture) stream, the second larger: the
    binding grows that stream's workspace for the second but keeps the first
    graph's, so replaying the first after the second still matches eager calls."""
    small = to_dev(wl.int_uniform(3 * 28672 + 5, 0, 16, seed=960))
    big = to_dev(wl.int_uniform(700 * 28672 + 7, 0, 16, seed=961))
    want_s = to_host(ps.scan_exclusive(small, "sum"))
    want_b = to_host(ps.scan_exclusive(big, "sum"))
    ys, yb = torch.empty_like(small), torch.empty_like(big)
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        ps.scan_exclusive(small, "sum", out=ys)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        ps.scan_exclusive(big, "sum", out=yb)
    for rep in range(3):
        ys.fill_(-1)
        yb.fill_(-1)
        g2.replay()
        g1.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(yb), want_b), f"replay {rep}: larger graph"
        assert np.array_equal(to_host(ys), want_s), f"replay {rep}: earlier graph"
        ps.scan_exclusive(big, "sum")  # eager work in between
        torch.cuda.synchronize()
