"""The block-level algorithms of the parallel prefix scan page, simulated step by
step in Python on its 8-element example, against the states the page prints
(geek-doc.cn, sections 二 and 三; the misprinted rows are corrected in the
fixtures, with the reason stated there).  These document the two algorithms the
block-scan kernels follow and the page errata; they do not involve the oracle."""
import numpy as np

from conftest import load_golden


def hillis_steele_states(x):
    """Each step k: every cell i >= 2^k adds the cell 2^k to its left, all cells
    reading the previous state (the double-buffered form)."""
    s = list(x)
    states, adds = [], 0
    k = 1
    while k < len(s):
        prev = list(s)
        for i in range(len(s)):
            if i >= k:
                s[i] = prev[i] + prev[i - k]
                adds += 1
        states.append(list(s))
        k *= 2
    return states, adds


def blelloch_states(x):
    s = list(x)
    n = len(s)
    ups, downs, adds = [], [], 0
    d = 1
    while d < n:
        for i in range(n):
            if (i + 1) % (2 * d) == 0:
                s[i] += s[i - d]
                adds += 1
        ups.append(list(s))
        d *= 2
    s[n - 1] = 0
    cleared = list(s)
    d = n // 2
    while d >= 1:
        for i in range(n):
            if (i + 1) % (2 * d) == 0:
                t = s[i - d]
                s[i - d] = s[i]
                s[i] += t
                adds += 1
        downs.append(list(s))
        d //= 2
    return ups, cleared, downs, adds


def test_hillis_steele_trace():
    g = load_golden("hillis_steele_trace.txt")
    states, _ = hillis_steele_states(g["x"])
    assert states == [g["after_stride_1"], g["after_stride_2"], g["after_stride_4"]]
    # the window rule: after the step with stride 2^k, cell i sums the window of
    # length 2^(k+1) ending at i
    x = g["x"]
    for k, st in enumerate(states):
        w = 2 ** (k + 1)
        assert st == [sum(x[max(0, i - w + 1):i + 1]) for i in range(len(x))]


def test_blelloch_trace():
    g = load_golden("blelloch_trace.txt")
    ups, cleared, downs, _ = blelloch_states(g["x"])
    assert ups == [g["up_d1"], g["up_d2"], g["up_d4"]]
    assert cleared == g["root_cleared"]
    assert downs == [g["down_d4"], g["down_d2"], g["down_d1"]]
    we = load_golden("worked_example.txt")
    assert downs[-1] == we["exclusive"]
    # the rule of the down-sweep: the value handed to a node is the sum of all
    # elements left of the node's range
    x = g["x"]
    assert downs[0][3] == 0 and downs[0][7] == sum(x[:4])


def test_work_and_depth_n1024():
    g = load_golden("op_counts_n1024.txt")
    n = g["n"][0]
    x = list(np.ones(n, dtype=np.int64))
    states, hs_adds = hillis_steele_states(x)
    assert len(states) == g["hs_steps"][0]
    assert hs_adds == g["hs_adds_exact"][0]
    ups, _, downs, bl_adds = blelloch_states(x)
    assert len(ups) + len(downs) == g["blelloch_steps"][0]
    assert bl_adds == g["blelloch_adds"][0]
    assert n - 1 == g["serial_adds"][0]
    assert states[-1] == list(range(1, n + 1))
    _, w_adds = hillis_steele_states(list(range(32)))
    assert len(hillis_steele_states(list(range(32)))[0]) == g["warp_steps_32"][0]
