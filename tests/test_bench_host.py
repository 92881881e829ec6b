"""Host-side logic of bench.py, on the CPU: the source digest that ties the recorded
HBM counters to the scan sources, the reading of those counters, the spread of the
timed batches, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_digest_ignores_comments_and_blank_lines():
    code = "int f(int x)\n{\n    return x + 1;  // one more\n}\n"
    commented = "/* a block\n   comment */\nint f(int x)\n{\n\n    // why\n    return x + 1;\n}\n"
    changed = "int f(int x)\n{\n    return x + 2;\n}\n"
    assert bench._code_only(code) == bench._code_only(commented)
    assert bench._code_only(code) != bench._code_only(changed)


def test_digest_follows_the_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() { }  // first\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.source_digest(["k.hip"])
    src.write_text("// a new comment\n__global__ void k() { }\n")
    assert bench.source_digest(["k.hip"]) == d0
    src.write_text("__global__ void k() { int a = 0; }\n")
    assert bench.source_digest(["k.hip"]) != d0


def test_recorded_traffic_matches_the_current_scan_sources():
    """The committed counters were taken from the current scan code: the bench reports
    them (about 1.0025 x the 2 GiB of one 2^28 scan)."""
    t = bench.read_traffic()
    assert t is not None
    assert 1.0 < t / (2 * (1 << 28) * 4) < 1.01


def test_traffic_is_null_for_other_sources(tmp_path, monkeypatch):
    with open(bench.PROFILE_TRAFFIC) as f:
        text = f.read()
    stale = tmp_path / "counters.txt"
    stale.write_text(text.replace("source_sha256_16: ", "source_sha256_16: 0"))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(stale))
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "missing.txt"))
    assert bench.read_traffic() is None


def test_spread_is_median_and_minimum_of_the_batches():
    t = bench.Timer(torch=None)
    t.batches = [0.3, 0.1, 0.2, 0.5, 0.4, 0.6]  # ms per call
    assert t.spread() == {"us_median": 400.0, "us_min": 100.0}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


class _FakeCuda:
    """Stands in for torch.cuda: events read a clock that every call advances."""

    def __init__(self):
        self.now_ms = 0.0
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1

    def Event(self, enable_timing=True):
        cuda = self

        class _Ev:
            def record(self):
                self.t = cuda.now_ms

            def elapsed_time(self, other):
                return other.t - self.t

        return _Ev()


class _FakeTorch:
    def __init__(self):
        self.cuda = _FakeCuda()


def test_legs_settle_before_the_timed_batches():
    """After the warmup calls a leg keeps calling, untimed, until the GPU has been busy
    for settle_ms; the timed batches then hold exactly `steps` calls each."""
    torch = _FakeTorch()
    calls = []

    def fn(i):
        calls.append(i)
        torch.cuda.now_ms += 0.1  # the call's GPU time
        bench.time.sleep(0.0005)

    t = bench.Timer(torch)
    ms = t.run(fn, steps=4, warmup=3, settle_ms=20.0)
    timed = 4 * (1 + bench.Timer.REPEATS)
    untimed = len(calls) - timed
    assert untimed > 3 + 8  # the warmup calls, then at least one round of settle calls
    assert (untimed - 3) % 8 == 0
    assert calls == list(range(untimed)) + list(range(4)) * (1 + bench.Timer.REPEATS)
    assert abs(ms - 0.1) < 1e-9
    assert len(t.batches) == 1 + bench.Timer.REPEATS


def test_headline_timing_takes_exactly_the_warmup_calls():
    torch = _FakeTorch()
    calls = []

    def fn(i):
        calls.append(i)
        torch.cuda.now_ms += 0.2

    bench.Timer(torch).run(fn, steps=5, warmup=7)
    assert len(calls) == 7 + 5 * (1 + bench.Timer.REPEATS)
