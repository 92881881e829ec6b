"""Benchmark of libscan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs scan,compact,...] [--settle-ms S]

A step is one device-wide int32 exclusive sum scan of N = 2^28 elements (values
U{0..15}), inputs resident in HBM.  The headline `value` is Gelem/s over exactly K
timed steps, bracketed by device synchronisation; HIP events on the stream the
library launches on give the time.  The JSON line also carries:
  roofline      achieved algorithmic HBM GB/s of the scan (2 * N * 4 bytes per
                step) against the 8 TB/s MI355X peak; `traffic` is the measured HBM
                bytes per launch from rocprofv3 counters (profiles/), or null when
                the kernel source changed since they were taken;
  cpu_baseline  the serial CPU oracle timed on this host on the same input, repeated
                for at least 10 s;
  legs          the other workloads: fused compaction (N = 2^27 at 1/50/99 %),
                float32 sum and int32 max scans (N = 2^26), the two batched row
                shapes, the 2^20 scan (latency-bound), and the plain read / write /
                copy kernels of libls_ceiling.so over the headline's bytes (the
                practical bandwidth ceilings).  A leg runs W warmup calls, then
                more untimed calls until the GPU has been busy for S ms (default 50;
                the host prepares each workload while the GPU idles), then six timed batches
                of K calls; it reports the first batch's mean and the median and
                minimum of the batch means, per call.
The benchmark runs on one GPU (rank 0); --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Each bandwidth leg keeps calling its workload, untimed, until the GPU has been busy
# this long after the warmup calls, before the timed batches start.
LEG_SETTLE_MS = 50.0
# The CPU oracle runs the headline workload over and over for at least this long.
CPU_BASELINE_S = 10.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "scan_i32_excl_n2e28_hbm_counters.txt")
SCAN_SOURCES = ["prefix_scan_stream_amd/csrc/ls_scan.hip", "prefix_scan_stream_amd/csrc/ls_device.hpp"]
ALL_LEGS = ("scan", "small", "fp32", "max", "compact", "rows64", "rows1024", "ceiling", "schemes",
            "blockscans", "sort", "select", "ops", "segmented")
DEFAULT_LEGS = ALL_LEGS


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments or blank lines, each line stripped: what the
    compiler sees, so that a change to a comment keeps the recorded counters."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).strip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
    same kernel source (calibrated against a plain copy), or None."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    kv = {}
    with open(PROFILE_TRAFFIC) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_digest(SCAN_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events recorded on the current stream, the one the library launches on.
    A run times `steps` calls between two events (the mean it returns), then
    repeats the same batch REPEATS more times for the spread: the median and
    minimum of the batch means.  (An event between every call would add a few
    microseconds to each.)"""

    REPEATS = 5

    def __init__(self, torch):
        self.torch = torch
        self.batches = []  # batch means (ms per step) of the last run

    def _batch(self, fn, steps: int) -> float:
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def run(self, fn, steps: int, warmup: int, settle_ms: float = 0.0) -> float:
        for i in range(warmup):
            fn(i)
        if settle_ms > 0:
            # more untimed calls until the GPU has been busy for settle_ms: after
            # the host-side preparation of a workload the GPU has idled for a while
            torch = self.torch
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            i = warmup
            while (time.perf_counter() - t0) * 1e3 < settle_ms:
                for _ in range(8):
                    fn(i)
                    i += 1
                torch.cuda.synchronize()
        ms = self._batch(fn, steps)
        self.batches = [ms] + [self._batch(fn, steps) for _ in range(self.REPEATS)]
        return ms  # ms per step of the first batch

    def spread(self) -> dict:
        """Median and minimum over the batches of the last run (us per call)."""
        t = sorted(self.batches)
        return {"us_median": round(1e3 * t[len(t) // 2], 2), "us_min": round(1e3 * t[0], 2)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.partition(":")[2].strip()
    except OSError:
        pass
    return "unknown"


class Ceilings:
    """The plain read / write / copy kernels of libls_ceiling.so (include/ls_ceiling.h)."""

    def __init__(self):
        import ctypes
        path = os.path.join(ROOT, "prefix_scan_stream_amd", "libls_ceiling.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} not found; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        P, SZ, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        lib.ls_ceiling_read.argtypes = [P, SZ, P, I, P]
        lib.ls_ceiling_write.argtypes = [P, SZ, I, P]
        lib.ls_ceiling_copy.argtypes = [P, P, SZ, I, P]
        self.lib = lib

    def call(self, kind, torch, a, b, sink, bpc):
        s = torch.cuda.current_stream().cuda_stream
        if kind == "read":
            st = self.lib.ls_ceiling_read(a.data_ptr(), a.numel() * a.element_size(), sink.data_ptr(), bpc, s)
        elif kind == "write":
            st = self.lib.ls_ceiling_write(b.data_ptr(), b.numel() * b.element_size(), bpc, s)
        else:
            st = self.lib.ls_ceiling_copy(a.data_ptr(), b.data_ptr(), a.numel() * a.element_size(), bpc, s)
        if st != 0:
            raise RuntimeError(f"ls_ceiling_{kind} returned {st}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--legs", default=",".join(DEFAULT_LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=LEG_SETTLE_MS,
                    help="untimed GPU-busy time of each leg after its warmup (0: none)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)
    legs = [s for s in args.legs.split(",") if s]
    for s in legs:
        if s not in ALL_LEGS:
            sys.exit(f"bench.py: unknown leg {s}; choose from {','.join(ALL_LEGS)}")

    import torch

    import prefix_scan_stream_amd as ps
    import workloads as wl

    if not torch.cuda.is_available():
        sys.exit("bench.py: no GPU visible")
    dev = torch.device("cuda:0")
    ps.load_library()  # fails loudly if the HIP library is missing
    timer = Timer(torch)
    K, W = args.steps, args.warmup
    result_legs = {}

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    headline = None
    if "scan" in legs:
        n = wl.SIZES["big_scan"]
        log(f"scan: generating int32 U{{0..15}} N={n}")
        x_host = wl.big_scan()
        x = to_dev(x_host)
        out = torch.empty_like(x)
        log(f"scan: {W} warmup + {K} timed steps")
        ms = timer.run(lambda i: ps.scan_exclusive(x, "sum", out=out), K, W)
        # one sampled correctness check of what was timed, against the oracle run below
        sample_idx = np.random.default_rng(1).integers(0, n, 4096)
        got_sample = out[torch.from_numpy(sample_idx).to(dev)].cpu().numpy()
        gelem = n / (ms * 1e-3) / 1e9
        algo_bytes = 2 * n * 4
        achieved = algo_bytes / (ms * 1e-3) / 1e9
        traffic = read_traffic()
        headline = dict(n=n, ms=ms, gelem=gelem, achieved=achieved, algo_bytes=algo_bytes,
                        traffic=traffic, **timer.spread())
        log(f"scan: {ms * 1e3:.1f} us/step, {gelem:.1f} Gelem/s, {achieved:.0f} GB/s")
        cpu = None
        if not args.no_cpu_baseline:
            import oracle
            log(f"scan: timing the CPU oracle on the same input (serial, 1 thread, "
                f"repeated for at least {CPU_BASELINE_S:.0f} s)")
            t0 = time.perf_counter()
            ref = oracle.scan(x_host, "sum", inclusive=False)
            ok = bool(np.array_equal(ref.y[sample_idx], got_sample))
            del ref
            reps = 1
            while time.perf_counter() - t0 < CPU_BASELINE_S:
                oracle.scan(x_host, "sum", inclusive=False)
                reps += 1
            t1 = time.perf_counter()
            cpu = {"value": round(reps * n / (t1 - t0) / 1e9, 4), "unit": "Gelem/s", "cores": 1,
                   "kind": "oracle",
                   "sample": f"the whole workload {reps} times: int32 exclusive sum of N={n} "
                             f"({t1 - t0:.1f} s on 1 of {len(os.sched_getaffinity(0))} host cores)",
                   "cpu_model": cpu_model(), "host_cores": len(os.sched_getaffinity(0))}
            headline["sample_check"] = ok
            if not ok:
                log("scan: SAMPLED OUTPUT DISAGREES WITH THE ORACLE")
        headline["cpu"] = cpu
        del x, out, x_host
        torch.cuda.empty_cache()

    def rotating(make, sets=3):
        return [make(i) for i in range(sets)]

    if "small" in legs:
        x = to_dev(wl.small_scan())
        out = torch.empty_like(x)
        ms = timer.run(lambda i: ps.scan_exclusive(x, "sum", out=out), max(K, 50), W)
        result_legs["small_scan_i32_excl_2e20"] = {"us": round(ms * 1e3, 2), **timer.spread(),
                                                   "gelem_s": round(x.numel() / ms / 1e6, 1),
                                                   "note": "cache-resident, latency-bound"}
        log(f"small: {ms * 1e3:.2f} us")

    def bw_leg(name, xs, fn, elems, nbytes):
        outs = [torch.empty_like(t) for t in xs]
        ms = timer.run(lambda i: fn(xs[i % len(xs)], outs[i % len(outs)]), K, W, settle_ms=args.settle_ms)
        gbs = nbytes / (ms * 1e-3) / 1e9
        result_legs[name] = {"us": round(ms * 1e3, 1), **timer.spread(),
                             "gelem_s": round(elems / ms / 1e6, 1), "algo_gbs": round(gbs, 1),
                             "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"{name}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")

    if "fp32" in legs:
        n = wl.SIZES["fp32_scan"]
        xs = rotating(lambda i: to_dev(wl.fp32_scan()))
        bw_leg("fp32_sum_incl_2e26", xs, lambda a, b: ps.scan_inclusive(a, "sum", out=b), n, 8 * n)
        # the fixed-order single pass: the same bits on every run
        bw_leg("fp32_sum_incl_2e26_deterministic", xs,
               lambda a, b: ps.scan_ex(a, "sum", True, "deterministic", out=b), n, 8 * n)
        del xs
    if "max" in legs:
        n = wl.SIZES["max_scan"]
        xs = rotating(lambda i: to_dev(wl.max_scan()))
        bw_leg("i32_max_incl_2e26", xs, lambda a, b: ps.scan_inclusive(a, "max", out=b), n, 8 * n)
        del xs
    if "compact" in legs:
        n = wl.SIZES["compact"]
        xh = wl.compact_input()
        xs = rotating(lambda i: to_dev(xh), sets=2)
        cnt = torch.empty(1, dtype=torch.int64, device=dev)
        for sel in wl.SELECTIVITIES:
            thr = wl.threshold_for(sel)
            kept = int(np.count_nonzero(xh < thr))
            bw_leg(f"compact_i32_2e27_sel{int(sel * 100)}", xs,
                   lambda a, b, thr=thr: ps.compact_if(a, "lt", thr, out=b, count=cnt), n,
                   4 * n + 4 * kept)
        del xs, xh
    if "select" in legs:
        # compaction by a byte flag array, and index selection, 2^27 elements, half kept
        n = wl.SIZES["compact"]
        xh = wl.compact_input()
        fh = (wl.u32_bits(n, seed=77) & 1).astype(np.uint8)
        kept = int(np.count_nonzero(fh))
        xs = rotating(lambda i: to_dev(xh), sets=2)
        fd = to_dev(fh)
        cnt = torch.empty(1, dtype=torch.int64, device=dev)
        bw_leg("compact_flags_i32_2e27_sel50", xs,
               lambda a, b: ps.compact_flags(a, fd, out=b, count=cnt), n, 5 * n + 4 * kept)
        bw_leg("select_indices_flags_2e27_sel50", xs,
               lambda a, b: ps.select_indices_flags(fd, out=b, count=cnt), n, n + 4 * kept)
        thr = wl.threshold_for(0.5)
        kept = int(np.count_nonzero(xh < thr))
        bw_leg("select_indices_if_i32_2e27_sel50", xs,
               lambda a, b: ps.select_indices_if(a, "lt", thr, out=b, count=cnt), n, 4 * n + 4 * kept)
        del xs, xh, fh, fd
    if "ops" in legs:
        # the further operators, inclusive scans of 2^26 elements
        n = wl.SIZES["fp32_scan"]
        for dt, op in (("int32", "min"), ("uint32", "or"), ("int32", "prod"), ("float32", "prod"),
                       ("uint32", "affine")):
            xs = rotating(lambda i, dt=dt, op=op: to_dev(wl.case(dt, op, n, seed=500 + i)))
            bw_leg(f"{dt}_{op}_incl_2e26", xs, lambda a, b, op=op: ps.scan_inclusive(a, op, out=b),
                   n, 8 * n)
            del xs
    if "segmented" in legs:
        # 2^26 int32 values in segments of random length (mean 1024), inclusive sums
        n = wl.SIZES["fp32_scan"]
        g = np.random.default_rng(wl.BASE_SEED + 50)
        hh = (g.random(n) < 1.0 / 1024).astype(np.uint8)
        hh[0] = 1
        offs = np.concatenate([np.flatnonzero(hh), [n]]).astype(np.int64)
        xs = rotating(lambda i: to_dev(wl.int_uniform(n, 0, 16, seed=700 + i)))
        hd, od = to_dev(hh), to_dev(offs)
        bw_leg("segmented_heads_i32_incl_2e26", xs,
               lambda a, b: ps.segmented_scan(a, "sum", False, heads=hd, out=b), n, 9 * n)
        bw_leg("segmented_offsets_i32_incl_2e26", xs,
               lambda a, b: ps.segmented_scan(a, "sum", False, offsets=od, out=b), n,
               8 * n + 8 * offs.size)
        del xs, hd, od
    if "rows64" in legs:
        xs = rotating(lambda i: to_dev(wl.rows64()))
        n = xs[0].numel()
        bw_leg("rows_2e20x64_f32_excl", xs, lambda a, b: ps.batched_row_scan(a, "sum", True, out=b),
               n, 8 * n)
        del xs
    if "rows1024" in legs:
        xs = rotating(lambda i: to_dev(wl.rows1024()))
        n = xs[0].numel()
        bw_leg("rows_2e16x1024_i32_excl", xs,
               lambda a, b: ps.batched_row_scan(a, "sum", True, out=b), n, 8 * n)
        del xs
    if "schemes" in legs:
        # the three-phase device schemes on the headline workload (same bytes in and out)
        n = wl.SIZES["big_scan"]
        x = to_dev(wl.big_scan())
        out = torch.empty_like(x)
        for scheme, moved in (("reduce_then_scan", 3), ("scan_then_propagate", 4)):
            ms = timer.run(lambda i, sc=scheme: ps.scan_ex(x, "sum", False, sc, out=out), K, W,
                           settle_ms=args.settle_ms)
            gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
            result_legs[f"scheme_{scheme}_i32_excl_2e28"] = {
                "us": round(ms * 1e3, 1), **timer.spread(), "gelem_s": round(n / ms / 1e6, 1),
                "algo_gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "bytes_moved_per_elem": 4 * moved}
            log(f"scheme {scheme}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s (algorithmic)")
        del x, out
    if "blockscans" in legs:
        # the block-level scan variants on 2^16 rows x 1024 int32 (one block per row)
        xs = rotating(lambda i: to_dev(wl.rows1024()))
        n = xs[0].numel()
        for kind in ("wave_dpp", "hillis_steele", "hillis_steele_double", "blelloch"):
            bw_leg(f"rows_2e16x1024_i32_excl_{kind}", xs,
                   lambda a, b, k=kind: ps.batched_row_scan_ex(a, "sum", True, k, out=b), n, 8 * n)
        del xs
    if "sort" in legs:
        # stable LSD radix sort (4 passes of 8 bits) of 2^24 uint32 keys, with and
        # without 32-bit values; per pass: histogram read, scatter read + write
        n = 1 << 24
        keys = to_dev(wl.u32_bits(n, seed=99))
        vals = torch.arange(n, dtype=torch.int32, device=dev)
        ok_, ov_ = torch.empty_like(keys), torch.empty_like(vals)
        for name, v, per_pass in (("sort_u32_pairs_2e24", vals, 20), ("sort_u32_keys_2e24", None, 12)):
            ms = timer.run(lambda i, v=v: ps.radix_sort(keys, v, out_keys=ok_,
                                                        out_values=ov_ if v is not None else None), K, W,
                           settle_ms=args.settle_ms)
            moved = 4 * per_pass * n
            result_legs[name] = {"us": round(ms * 1e3, 1), **timer.spread(), "gkeys_s": round(n / ms / 1e6, 2),
                                 "moved_gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                                 "bytes_moved_per_key": 4 * per_pass}
            log(f"{name}: {ms * 1e3:.1f} us (median {timer.spread()['us_median']}), {n / ms / 1e6:.2f} Gkeys/s")
        del keys, vals, ok_, ov_
    if "ceiling" in legs:
        # plain read / write / copy kernels over the headline's bytes (1 GiB each way):
        # the practical ceilings, best over three grid sizes
        n = wl.SIZES["big_scan"]
        a = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
        b = torch.empty_like(a)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        ce = Ceilings()
        for kind, nbytes in (("read", 4 * n), ("write", 4 * n), ("copy", 8 * n)):
            best = None
            for bpc in (4, 8, 16):
                ms = timer.run(lambda i, k=kind, bpc=bpc: ce.call(k, torch, a, b, sink, bpc), K, W,
                               settle_ms=args.settle_ms)
                if best is None or ms < best[0]:
                    best = (ms, bpc, timer.spread())
            ms, bpc, spread = best
            gbs = nbytes / (ms * 1e-3) / 1e9
            result_legs[f"ceiling_{kind}_1GiB"] = {"us": round(ms * 1e3, 1), **spread, "gbs": round(gbs, 1),
                                                  "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                                                  "blocks_per_cu": bpc}
            log(f"ceiling {kind}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s ({bpc} blocks per CU)")
        del a, b

    if headline is None:
        print(json.dumps({"legs": result_legs}))
        return
    h = headline
    line = {
        "metric": "int32 exclusive scan Gelem/s + HBM GB/s (% of peak) at N=2^28; compact Gelem/s",
        "value": round(h["gelem"], 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(h["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": "int32 exclusive sum scan, N=2^28, values U{0..15} (numpy PCG64)",
                   "n": h["n"], "scheme": "single pass, tile prefixes published by one chasing wave",
                   "tile_elems": 28672},
        "roofline": {"bound": "hbm", "achieved": round(h["achieved"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(h["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": h["traffic"]},
        "step_us": {"mean": round(h["ms"] * 1e3, 2), "median": h["us_median"], "min": h["us_min"]},
        "cpu_baseline": h["cpu"],
        "sample_check": h.get("sample_check"),
        "legs": result_legs,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
