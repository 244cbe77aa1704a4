#!/usr/bin/env python3
"""Throughput of the teacher-forced logit comparison on one MI355X.

One step = one pass of the whole path over one batch of synthetic positions:
lcmp_compare_logits with the bitwise statistics fused (streaming pass + per-row
finalize) followed by lcmp_bin_report (margin bins).  The default workload is
the scored-corpus shape: N=10240 positions x V=151936, fp32 baseline, bf16
candidate, k=20, six margin bins.  Inputs are generated on the host, copied to
HBM once, and are resident before the timed region starts.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      positions per second over the timed steps (whole job, one GPU)
  roofline   HBM roofline of the streaming kernel: algorithmic bytes per launch
             (N*V*(bytes per baseline + candidate element)) / its average
             duration, measured with HIP events recorded around that kernel on
             its own stream; traffic = measured HBM bytes per launch from the
             rocprofv3 FETCH_SIZE / WRITE_SIZE counters (copy-calibrated) when
             they were taken on the current kernel source, else null
  cpu_baseline  the double-precision CPU oracle on a bounded row sample

With --path record the step is instead the comparison against a compact
record of the baseline (lcmp_compare_record + lcmp_bin_report): the record is
made once before the timed region, and the streaming kernel reads only the
candidate rows (N*V*(bytes per candidate element) per launch).

Flags: --gpus N (only 1 is supported: this path runs on one GPU),
--steps K, --warmup W, --workload {corpus,segment,stream,tiny},
--path {compare,record},
--cpu-seconds S (budget of the oracle leg), --no-cpu-baseline,
--copy-probe BYTES (run only a plain device copy of that size, for counter
calibration under rocprofv3).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "logit positions/sec at V=151936 + achieved HBM GB/s vs MI355X peak"
# per path: the dominant kernel, its committed counter summary and its sources
PATHS = {
    "compare": dict(kernel="k_row_stats",
                    counters=os.path.join(ROOT, "profiles", "k_row_stats_corpus_counters.md"),
                    sources=("k_row_stats.hip", "common.hpp", "dma.hpp")),
    "record": dict(kernel="k_rest_sum",
                   counters=os.path.join(ROOT, "profiles", "k_rest_sum_corpus_counters.md"),
                   sources=("k_rest_sum.hip", "common.hpp", "dma.hpp")),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(path: str = "compare") -> str:
    h = hashlib.sha256()
    for name in PATHS[path]["sources"]:
        with open(os.path.join(ROOT, "logit_distribution_diffing_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, path: str = "compare"):
    """HBM bytes per launch of the path's streaming kernel from the committed
    counter summary, if it was taken on this kernel source and workload."""
    counters = PATHS[path]["counters"]
    if not os.path.exists(counters):
        return None
    text = open(counters).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_hash") != kernel_hash(path) or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


class Hip:
    """The few HIP runtime calls the timing needs (same runtime torch uses)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def make_inputs(workload: str, w: dict, torch):
    """Generate the workload on the host in row blocks and copy it to HBM.
    Returns device tensors plus a host copy of the first rows (CPU leg)."""
    import numpy as np
    import synth
    n, v = w["n"], w["v"]
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    base = torch.empty((n, v), dtype=dt[w["base"]], device="cuda")
    cand = torch.empty((n, v), dtype=dt[w["cand"]], device="cuda")
    keep = min(n, 16384)
    host_a = host_b = None
    blk = 1024
    t0 = time.time()
    for r0 in range(0, n, blk):
        nr = min(blk, n - r0)
        if workload == "tiny":
            a, b = synth.tiny(w["seed"], r0, nr, v)
        elif workload == "segment":
            a, b = synth.segment(w["seed"], r0, nr, v)
        elif workload == "corpus":
            a, b = synth.corpus(w["seed"], r0, nr, v, n, w["swap_frac"])
        elif workload == "stream":
            a, b = synth.stream(w["seed"], r0, nr, v)
        else:
            raise ValueError(workload)
        if r0 < keep:
            ka = a[: keep - r0]
            kb = b[: keep - r0]
            host_a = ka.copy() if host_a is None else np.concatenate([host_a, ka])
            host_b = kb.copy() if host_b is None else np.concatenate([host_b, kb])
        for dst, src in ((base, a), (cand, b)):
            t = torch.from_numpy(src.view(np.int16) if src.dtype == np.uint16 else src)
            dst[r0:r0 + nr].view(torch.int16 if src.dtype == np.uint16 else dst.dtype).copy_(t)
    torch.cuda.synchronize()
    log(f"[bench] generated and uploaded {workload} {n}x{v} in {time.time() - t0:.1f}s")
    return base, cand, host_a, host_b


def cpu_leg(host_a, host_b, k, edges, seconds: float):
    """Time the oracle (compare + bitwise + bins) on a bounded sample of rows."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows_avail = host_a.shape[0]
    probe = min(rows_avail, max(threads, 16))
    t0 = time.perf_counter()
    oracle.compare(host_a[:probe], host_b[:probe], k=k, nthreads=threads)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(probe, min(rows_avail, seconds / max(per_row, 1e-9))))
    t0 = time.perf_counter()
    o = oracle.compare(host_a[:rows], host_b[:rows], k=k, nthreads=threads)
    oracle.bitdiff(host_a[:rows], host_b[:rows], nthreads=threads)
    oracle.bin_report(o["margin"], o["flip"], o["kl_topk"], o["kl_full"], edges,
                      status=o["status"])
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="positions/s", cores=threads, kind="oracle",
                sample=f"first {rows} positions of the workload (compare + bitwise + bins), "
                       f"{dt:.1f} s")


def cpu_leg_record(host_a, host_b, k, edges, seconds: float):
    """Time the oracle's comparison against a record (+ bins) on a bounded sample
    of rows; the sample's record is made first, outside the timing, as the
    record of a baseline is made once."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows_avail = host_a.shape[0]
    probe = min(rows_avail, max(threads, 16))
    rec = oracle.record(host_a[:probe], k=k, nthreads=threads)
    t0 = time.perf_counter()
    oracle.compare_record(rec, host_b[:probe], k=k, nthreads=threads)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(probe, min(rows_avail, seconds / max(per_row, 1e-9))))
    rec = oracle.record(host_a[:rows], k=k, nthreads=threads)
    t0 = time.perf_counter()
    o = oracle.compare_record(rec, host_b[:rows], k=k, nthreads=threads)
    oracle.bin_report(o["margin"], o["flip"], o["kl_topk"], None, edges, status=o["status"])
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="positions/s", cores=threads, kind="oracle",
                sample=f"first {rows} positions of the workload (comparison against their "
                       f"record + bins), {dt:.1f} s")


def copy_probe(nbytes: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "dispatches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the first ~15 launches run while the clocks settle under the load, so
    # the default warm-up covers them
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="corpus", choices=["corpus", "segment", "stream", "tiny"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0)
    ap.add_argument("--path", default="compare", choices=["compare", "record"],
                    help="compare: baseline and candidate rows, full comparison (default); "
                         "record: the candidate against a compact record of the baseline, "
                         "made once before the timed steps")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this comparison path runs on one GPU; --gpus must be 1 "
              f"(got --gpus {args.gpus}, WORLD_SIZE {world}). Rows shard across GPUs "
              "with no exchange but the bin report; that mode is not built here.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    import synth
    import logit_distribution_diffing_amd as L

    w = dict(synth.WORKLOADS[args.workload])
    n, v, k = w["n"], w["v"], w["k"]
    edges = list(synth.DEFAULT_EDGES)
    base, cand, host_a, host_b = make_inputs(args.workload, w, torch)
    esize = {"f32": 4, "bf16": 2}
    hip = Hip()
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    stream = torch.cuda.current_stream()
    bws = torch.empty(int(L.lib().lcmp_bin_workspace_bytes(n, 1, len(edges))), dtype=torch.uint8,
                      device="cuda")
    bins = torch.empty((len(edges), L.BIN_BYTES), dtype=torch.uint8, device="cuda")
    summ = torch.empty((1, L.GROUP_SUMMARY_BYTES), dtype=torch.uint8, device="cuda")

    if args.path == "compare":
        # the streaming kernel reads both rows once
        bytes_per_launch = n * v * (esize[w["base"]] + esize[w["cand"]])
        out = L.alloc_compare_outputs(n, k, base.device, with_bitdiff=True)
        ws = torch.empty(L.compare_workspace_bytes(n, v, k, True), dtype=torch.uint8,
                         device="cuda")

        def step(ev=None):
            L.lcmp_compare_logits(base, cand, k=k, with_bitdiff=True, out=out, workspace=ws,
                                  stream=stream, events=ev)
            L.lcmp_bin_report(out["margin"], out["flip"], out["kl_topk"], out["kl_full"], edges,
                              status=out["status"], workspace=bws, stream=stream, bins=bins,
                              summary=summ)
    else:
        # the baseline is recorded once; the timed steps read the candidate rows
        # and the record only
        record = L.lcmp_record_baseline(base, k_rec=k)
        torch.cuda.synchronize()
        del base
        torch.cuda.empty_cache()
        bytes_per_launch = n * v * esize[w["cand"]]
        out = L.alloc_compare_outputs(n, k, cand.device)
        del out["kl_full"]
        ws = torch.empty(int(L.lib().lcmp_compare_record_workspace_bytes(n, v)),
                         dtype=torch.uint8, device="cuda")

        def step(ev=None):
            L.lcmp_compare_record(record, cand, k=k, out=out, workspace=ws, stream=stream,
                                  events=ev)
            L.lcmp_bin_report(out["margin"], out["flip"], out["kl_topk"], None, edges,
                              status=out["status"], workspace=bws, stream=stream, bins=bins,
                              summary=summ)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_stop)
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    kern_avg_s = sum(kern_ms) / len(kern_ms) / 1e3
    ms_per_step = gpu_ms / args.steps
    srt = sorted(kern_ms)
    log(f"[bench] {args.steps} steps: {gpu_ms:.3f} ms on the stream, {wall * 1e3:.3f} ms wall; "
        f"streaming kernel avg {kern_avg_s * 1e6:.1f} us (min {srt[0] * 1e3:.1f}, median "
        f"{srt[len(srt) // 2] * 1e3:.1f}, max {srt[-1] * 1e3:.1f} us; first five "
        f"{[round(x * 1e3) for x in kern_ms[:5]]})")

    b_np, s_np = L.unpack_bins(bins, summ)
    log(f"[bench] bins count {list(b_np[0]['count'])} flips {list(b_np[0]['flips'])} "
        f"big-margin flips {int(s_np[0]['big_margin_flips'])}")

    achieved = bytes_per_launch / kern_avg_s / 1e9
    traffic = stored_traffic(args.workload, args.path)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=PATHS[args.path]["kernel"], bytes_per_launch=bytes_per_launch)

    cpu = None
    if not args.no_cpu_baseline and host_a is not None:
        leg = cpu_leg if args.path == "compare" else cpu_leg_record
        cpu = leg(host_a, host_b, k, edges, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.1f} positions/s on {cpu['cores']} threads")

    value = n * args.steps / (gpu_ms / 1e3)
    wdesc = {
        "corpus": "scored corpus: 10240 positions (5 depths x 4 segments x 512) x V=151936, "
                  "fp32 baseline / bf16 candidate",
        "segment": "decoded segment: 512 positions x V=151936, fp32 / fp32",
        "stream": "large stream: 65536 positions x V=151936, bf16 / bf16",
        "tiny": "tiny compare: 64 positions x V=1024, fp32 / fp32",
    }[args.workload]
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wdesc, "path": args.path, "n": n, "v": v, "k": k,
                   "base": w["base"], "cand": w["cand"],
                   "bitwise_stats": args.path == "compare", "margin_edges": len(edges),
                   "hbm_gbs_step": round(bytes_per_launch / (ms_per_step / 1e3) / 1e9, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
