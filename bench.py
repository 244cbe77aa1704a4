#!/usr/bin/env python3
"""Throughput of the teacher-forced logit comparison on one MI355X.

One step = one pass of the whole path over one batch of synthetic positions:
lcmp_compare_logits with the bitwise statistics fused (streaming pass + per-row
finalize) followed by lcmp_bin_report (margin bins; on the corpus, per context
depth x code/prose group).  The default workload is the scored-corpus shape:
N=10240 positions x V=151936, fp32 baseline, bf16 candidate, k=20, six margin
bins, ten row groups.  Inputs are generated on the host, copied to HBM once,
and are resident before the timed region starts.

After W warm-up steps the K steps are timed in three passes, each between
synchronisations:
  1. one after the other on one stream, as one caller's stream runs them:
     roofline.ms_per_step_one_stream;
  2. on --streams S streams in turn (default 2), each stream with its own
     outputs and workspaces, as a caller scoring a sequence of batches would
     issue them: consecutive batches overlap, so one batch's latency-bound
     per-row finalize and bin report (and the ramp and tail of its streaming
     pass) run beside the next batch's streaming pass.  value and ms_per_step
     (time per batch) come from this pass (with --streams 1 it repeats pass 1);
  3. one after the other on one stream, with HIP events given to the dispatch
     of each step's streaming kernel: the kernel's duration (kernel_us), and
     roofline.ms_per_step_timed_pass (timing events leave the stream idle for
     a few microseconds around the kernel they time).
Kernel durations always come from pass 3, where no two kernels overlap.  With
a short warm-up the first launches after it still run slower while the clocks
settle, so the passes that give the figures come after a full pass.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      positions per second over the timed steps of pass 2 (whole job,
             one GPU)
  roofline   HBM roofline of the streaming kernel: algorithmic bytes per launch
             (N*V*(bytes per baseline + candidate element)) / its average
             duration over the event-timed pass (3).  Also: the same bytes over the
             whole step, and over
             the duration of a read-only stream of the same inputs in the same
             access pattern (lcmp_read_probe), the read rate this pattern can
             reach.  The probe runs before the warm-up steps; its untimed
             launches (at least 0.2 s) also take the clocks from idle to their
             loaded state, so the first timed steps do not run on ramping
             clocks.  traffic = measured HBM bytes per launch from the rocprofv3
             FETCH_SIZE / WRITE_SIZE counters (copy-calibrated), taken from the
             committed counter summary when it was measured on the current
             kernel source and workload (traffic_source says which file), else
             null
  cpu_baseline  the double-precision CPU oracle on a bounded row sample, with
             the host's CPU model; on the tiny and segment workloads also on one
             core

With --path record the step is instead the comparison against a compact
record of the baseline (lcmp_compare_record + lcmp_bin_report): the record is
made once before the timed region, and the streaming kernel reads only the
candidate rows (N*V*(bytes per candidate element) per launch).

--workload sweep times the bitwise / ULP mode over a shape sweep instead: one
step is lcmp_bitdiff over bf16 [T, 5120] for T in {1, 17, 65, 1024, 1502, 1777,
4095, 4096} and over fp32 [512, 151936] logit rows (rows/s and GB/s).

On the segment and sweep workloads (inputs below a few GB) the step rotates
over several copies of the inputs (--copies), so a step never finds its
inputs in the 256 MB last-level cache from the step before.

Flags: --gpus N (only 1 is supported: this path runs on one GPU),
--steps K, --warmup W, --workload {corpus,segment,stream,tiny,sweep},
--path {compare,record}, --copies C, --cpu-seconds S (budget of the oracle
leg), --no-cpu-baseline, --no-read-probe, --streams S,
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
SWEEP_METRIC = "bitwise rows/sec over the [T,5120] bf16 shape sweep and [512,151936] fp32 rows " \
               "+ achieved HBM GB/s vs MI355X peak"
# per path: the dominant kernel, its committed counter summaries (per workload)
# and its sources
PATHS = {
    "compare": dict(kernel="k_row_stats", prefix="k_row_stats",
                    sources=("k_row_stats.hip", "common.hpp", "dma.hpp")),
    "record": dict(kernel="k_rest_sum", prefix="k_rest_sum",
                   sources=("k_rest_sum.hip", "common.hpp", "dma.hpp")),
}
COPIES = {"corpus": 1, "stream": 1, "tiny": 1, "segment": 4, "sweep": 4}
WORKLOAD_DESC = {
    "corpus": "scored corpus: 10240 positions (5 depths x 4 segments x 512) x V=151936, "
              "fp32 baseline / bf16 candidate",
    "segment": "decoded segment: 512 positions x V=151936, fp32 / fp32",
    "stream": "large stream: 65536 positions x V=151936, bf16 / bf16",
    "tiny": "tiny compare: 64 positions x V=1024, fp32 / fp32",
    "sweep": "bitwise shape sweep: bf16 [T,5120] for T in {1,17,65,1024,1502,1777,4095,4096} "
             "plus fp32 [512,151936] logit rows, 0.1% of elements moved by 1-3 ULP",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(path: str = "compare") -> str:
    h = hashlib.sha256()
    for name in PATHS[path]["sources"]:
        with open(os.path.join(ROOT, "logit_distribution_diffing_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_file(workload: str, path: str = "compare") -> str:
    return os.path.join(ROOT, "profiles", f"{PATHS[path]['prefix']}_{workload}_counters.md")


def stored_traffic(workload: str, path: str = "compare"):
    """(HBM bytes per launch of the path's streaming kernel, the summary file)
    from the committed counter summary, if it was taken on this kernel source
    and workload; else (None, None)."""
    counters = counters_file(workload, path)
    if not os.path.exists(counters):
        return None, None
    text = open(counters).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None, None
    rec = json.loads(m.group(1))
    if rec.get("kernel_hash") != kernel_hash(path) or rec.get("workload") != workload:
        return None, None
    return rec.get("traffic_bytes_per_launch"), os.path.relpath(counters, ROOT)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


class Hip:
    """The few HIP runtime calls the timing needs (same runtime torch uses).

    The events are created with hipEventDisableSystemFence: they only time,
    and the flag leaves out the system-scope cache writeback and invalidation
    that a default event adds to the stream (on MI355X the idle gap around a
    timed kernel drops from about 5.6 to 4.5 us)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def stats_us(ms_list):
    srt = sorted(ms_list)
    return dict(mean=1e3 * sum(srt) / len(srt), median=1e3 * srt[len(srt) // 2],
                min=1e3 * srt[0], max=1e3 * srt[-1])


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
        if (r0 // blk) % 16 == 15:
            log(f"[bench] generated {r0 + nr}/{n} rows")
    torch.cuda.synchronize()
    log(f"[bench] generated and uploaded {workload} {n}x{v} in {time.time() - t0:.1f}s")
    return base, cand, host_a, host_b


def _bounded_rows(run, rows_avail, seconds, probe):
    """Rows of a sample that takes about `seconds`, from a timed probe of
    `probe` rows."""
    t0 = time.perf_counter()
    run(probe)
    per_row = (time.perf_counter() - t0) / probe
    return int(max(probe, min(rows_avail, seconds / max(per_row, 1e-9))))


def cpu_leg(host_a, host_b, k, edges, seconds: float, single_core: bool):
    """Time the oracle (compare + bitwise + bins) on a bounded sample of rows."""
    import oracle
    threads = oracle_threads()

    def run(rows, nthreads):
        o = oracle.compare(host_a[:rows], host_b[:rows], k=k, nthreads=nthreads)
        oracle.bitdiff(host_a[:rows], host_b[:rows], nthreads=nthreads)
        oracle.bin_report(o["margin"], o["flip"], o["kl_topk"], o["kl_full"], edges,
                          status=o["status"])

    rows_avail = host_a.shape[0]
    rows = _bounded_rows(lambda r: run(r, threads), rows_avail, seconds,
                         min(rows_avail, max(threads, 16)))
    t0 = time.perf_counter()
    run(rows, threads)
    dt = time.perf_counter() - t0
    res = dict(value=rows / dt, unit="positions/s", cores=threads, kind="oracle",
               sample=f"first {rows} positions of the workload (compare + bitwise + bins), "
                      f"{dt:.1f} s", cpu=cpu_model())
    if single_core:
        rows1 = _bounded_rows(lambda r: run(r, 1), rows_avail, seconds / 3, min(rows_avail, 4))
        t0 = time.perf_counter()
        run(rows1, 1)
        dt1 = time.perf_counter() - t0
        res["single_core"] = dict(value=rows1 / dt1, unit="positions/s", cores=1,
                                  sample=f"first {rows1} positions, {dt1:.1f} s")
    return res


def cpu_leg_record(host_a, host_b, k, edges, seconds: float):
    """Time the oracle's comparison against a record (+ bins) on a bounded sample
    of rows; the sample's record is made first, outside the timing, as the
    record of a baseline is made once."""
    import oracle
    threads = oracle_threads()
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
                       f"record + bins), {dt:.1f} s", cpu=cpu_model())


def copy_probe(nbytes: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "dispatches": 5}), flush=True)


def time_steps(step, steps, warmup, hip, torch, stream, lanes, nev=1):
    """Warm-up and timed passes of K steps.  step(i, evs, lane) runs step i on
    lane `lane`: one of len(lanes) streams, each with its own outputs and
    workspaces; `evs` (None outside the event pass) gives `nev` HIP event
    pairs to the dispatch of the step's streaming kernel(s).

    W untimed warm-up steps (on the lanes in turn), then, each pass between
    synchronisations on `stream`:
      1. the K steps one after the other on lane 0, as one stream runs them;
      2. the K steps on the lanes in turn (step i on lane i mod S): with more
         than one lane consecutive batches overlap, so one batch's per-row
         finalize and bin report run beside the next batch's streaming pass;
      3. the event pass: the K steps one after the other on lane 0, with
         events; their durations are the kernel times (a timed kernel leaves
         the stream idle for a few microseconds around it).
    With the driver's short warm-up the first launches after it still run
    slower (the clocks settle over some tens of launches), so the event pass
    comes last and the pass that gives the value comes after a full pass.
    Returns the stream time of the value pass (2) (ms), its wall time (s), per
    event pair the list of its K durations (ms), and the stream times of
    passes 3 and 1 (ms)."""
    nl = len(lanes)
    for i in range(warmup):
        step(i, None, i % nl)
    torch.cuda.synchronize()

    def timed(first, evs, pipelined):
        t_start = torch.cuda.Event(enable_timing=True)
        t_stop = torch.cuda.Event(enable_timing=True)
        used = lanes if pipelined else lanes[:1]
        wall0 = time.perf_counter()
        t_start.record(stream)
        for s_ in used:
            s_.wait_stream(stream)
        for i in range(steps):
            step(first + i, evs and evs[i], i % nl if pipelined else 0)
        for s_ in used:
            stream.wait_stream(s_)
        t_stop.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_stop), time.perf_counter() - wall0

    one_ms, _ = timed(warmup, None, False)
    gpu_ms, wall = timed(warmup + steps, None, True)
    evs = [[(hip.event(), hip.event()) for _ in range(nev)] for _ in range(steps)]
    ev_ms, _ = timed(warmup + 2 * steps, evs, False)
    per = [[hip.elapsed_ms(a, b) for a, b in (evs[i][j] for i in range(steps))]
           for j in range(nev)]
    return gpu_ms, wall, per, ev_ms, one_ms


def read_ceiling(L, pairs, hip, torch, stream, reps=12, settle_s=0.2):
    """Median duration (us) of the read-only probe over the same inputs (the
    copies in turn).  Untimed launches come first, for at least settle_s
    seconds of wall time: the probe runs before the timed steps, and these
    launches also bring the GPU clocks from idle to their loaded state."""
    base0, cand0 = pairs[0]
    ws = torch.empty(int(L.lib().lcmp_compare_workspace_bytes(base0.size(0), base0.size(1), 1, 0)),
                     dtype=torch.uint8, device="cuda")
    i = 0
    t0 = time.perf_counter()
    while i < 3 or time.perf_counter() - t0 < settle_s:
        for _ in range(4):
            base, cand = pairs[i % len(pairs)]
            L.lcmp_read_probe(base, cand, workspace=ws, stream=stream)
            i += 1
        torch.cuda.synchronize()
    ms = []
    for j in range(reps):
        base, cand = pairs[(i + j) % len(pairs)]
        ev = (hip.event(), hip.event())
        L.lcmp_read_probe(base, cand, workspace=ws, stream=stream, events=ev)
        ms.append(ev)
    torch.cuda.synchronize()
    return stats_us([hip.elapsed_ms(a, b) for a, b in ms])


def run_compare(args, torch, L, synth):
    w = dict(synth.WORKLOADS[args.workload])
    n, v, k = w["n"], w["v"], w["k"]
    edges = list(synth.DEFAULT_EDGES)
    base, cand, host_a, host_b = make_inputs(args.workload, w, torch)
    copies = args.copies or COPIES[args.workload]
    pairs = [(base, cand)] + [(base.clone(), cand.clone()) for _ in range(copies - 1)]
    esize = {"f32": 4, "bf16": 2}
    hip = Hip()
    stream = torch.cuda.current_stream()
    if args.workload == "corpus":
        groups = torch.from_numpy(synth.corpus_groups(n)).cuda()
        n_groups = synth.CORPUS_GROUPS
    else:
        groups, n_groups = None, 1
    lanes = [torch.cuda.Stream() for _ in range(args.streams)]  # default priority
    bin_sets = [dict(bws=torch.empty(int(L.lib().lcmp_bin_workspace_bytes(n, n_groups, len(edges))),
                                     dtype=torch.uint8, device="cuda"),
                     bins=torch.empty((n_groups * len(edges), L.BIN_BYTES), dtype=torch.uint8,
                                      device="cuda"),
                     summ=torch.empty((n_groups, L.GROUP_SUMMARY_BYTES), dtype=torch.uint8,
                                      device="cuda")) for _ in lanes]

    if args.path == "compare":
        # the streaming kernel reads both rows once
        bytes_per_launch = n * v * (esize[w["base"]] + esize[w["cand"]])
        outs = [L.alloc_compare_outputs(n, k, base.device, with_bitdiff=True) for _ in lanes]
        wss = [torch.empty(L.compare_workspace_bytes(n, v, k, True), dtype=torch.uint8,
                           device="cuda") for _ in lanes]

        def step(i, evs, lane):
            b_, c_ = pairs[i % copies]
            out, z, s_ = outs[lane], bin_sets[lane], lanes[lane]
            L.lcmp_compare_logits(b_, c_, k=k, with_bitdiff=True, out=out, workspace=wss[lane],
                                  stream=s_, events=evs and evs[0])
            L.lcmp_bin_report(out["margin"], out["flip"], out["kl_topk"], out["kl_full"], edges,
                              status=out["status"], group=groups, n_groups=n_groups,
                              workspace=z["bws"], stream=s_, bins=z["bins"], summary=z["summ"])
    else:
        # the baseline is recorded once; the timed steps read the candidate rows
        # and the record only
        record = L.lcmp_record_baseline(base, k_rec=k)
        torch.cuda.synchronize()
        bytes_per_launch = n * v * esize[w["cand"]]
        outs = []
        for _ in lanes:
            o_ = L.alloc_compare_outputs(n, k, cand.device)
            del o_["kl_full"]
            outs.append(o_)
        wss = [torch.empty(int(L.lib().lcmp_compare_record_workspace_bytes(n, v)),
                           dtype=torch.uint8, device="cuda") for _ in lanes]

        def step(i, evs, lane):
            c_ = pairs[i % copies][1]
            out, z, s_ = outs[lane], bin_sets[lane], lanes[lane]
            L.lcmp_compare_record(record, c_, k=k, out=out, workspace=wss[lane], stream=s_,
                                  events=evs and evs[0])
            L.lcmp_bin_report(out["margin"], out["flip"], out["kl_topk"], None, edges,
                              status=out["status"], group=groups, n_groups=n_groups,
                              workspace=z["bws"], stream=s_, bins=z["bins"], summary=z["summ"])

    # the read-only probe first: its untimed launches settle the clocks
    probe = None
    if not args.no_read_probe and args.path == "compare":
        probe = read_ceiling(L, pairs, hip, torch, stream)
    gpu_ms, wall, (kern_ms,), ev_ms, one_ms = time_steps(step, args.steps, args.warmup, hip,
                                                         torch, stream, lanes)
    ks = stats_us(kern_ms)
    ms_per_step = gpu_ms / args.steps
    log(f"[bench] {args.steps} steps on {len(lanes)} stream(s): {gpu_ms:.3f} ms, "
        f"{wall * 1e3:.3f} ms wall; on one stream {one_ms:.3f} ms, with timing events "
        f"{ev_ms:.3f} ms; streaming kernel mean {ks['mean']:.1f} us, "
        f"median {ks['median']:.1f} (min {ks['min']:.1f}, max {ks['max']:.1f}); first five "
        f"{[round(x * 1e3) for x in kern_ms[:5]]} us; input copies in turn: {copies}")
    b_np, s_np = L.unpack_bins(bin_sets[0]["bins"], bin_sets[0]["summ"], n_groups)
    log(f"[bench] bins count {b_np['count'].sum(axis=0).tolist()} flips "
        f"{b_np['flips'].sum(axis=0).tolist()} big-margin flips "
        f"{int(s_np['big_margin_flips'].sum())} over {n_groups} group(s)")

    if probe is not None:
        log(f"[bench] read-only probe of the same pattern: median {probe['median']:.1f} us "
            f"({bytes_per_launch / probe['median'] / 1e3:.1f} GB/s)")

    gbs = lambda us: round(bytes_per_launch / us / 1e3, 1)  # noqa: E731
    achieved = gbs(ks["mean"])
    traffic, traffic_src = stored_traffic(args.workload, args.path)
    roofline = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    traffic_source=(f"{traffic_src}: rocprofv3 FETCH_SIZE + WRITE_SIZE of this "
                                    "kernel source, copy-calibrated" if traffic_src else None),
                    kernel=PATHS[args.path]["kernel"], bytes_per_launch=bytes_per_launch,
                    kernel_us=dict((key, round(val, 1)) for key, val in ks.items()),
                    achieved_median=gbs(ks["median"]),
                    step_achieved=gbs(1e3 * ms_per_step),
                    step_frac=round(gbs(1e3 * ms_per_step) / HBM_PEAK_GBS, 4),
                    ms_per_step_one_stream=round(one_ms / args.steps, 4),
                    ms_per_step_timed_pass=round(ev_ms / args.steps, 4))
    if probe is not None:
        roofline["read_ceiling"] = gbs(probe["median"])
        roofline["frac_of_read_ceiling"] = round(achieved / gbs(probe["median"]), 4)

    cpu = None
    if not args.no_cpu_baseline and host_a is not None:
        if args.path == "compare":
            cpu = cpu_leg(host_a, host_b, k, edges, args.cpu_seconds,
                          single_core=args.workload in ("tiny", "segment"))
        else:
            cpu = cpu_leg_record(host_a, host_b, k, edges, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.1f} positions/s on {cpu['cores']} threads "
            f"({cpu['cpu']})")

    value = n * args.steps / (gpu_ms / 1e3)
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "path": args.path, "n": n, "v": v,
                   "k": k, "base": w["base"], "cand": w["cand"],
                   "arithmetic": "fp32 per element, fp64 sums and finalize",
                   "bitwise_stats": args.path == "compare", "margin_edges": len(edges),
                   "row_groups": n_groups, "input_copies": copies, "streams": len(lanes),
                   "hbm_gbs_step": roofline["step_achieved"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


def run_sweep(args, torch, L, synth):
    """Bitwise / ULP mode over the shape sweep: one step = lcmp_bitdiff over
    every shape of the sweep, the fp32 logit rows last."""
    import numpy as np
    w = synth.WORKLOADS["sweep"]
    cols, v, frac, seed = w["cols"], w["v"], w["frac"], w["seed"]
    t0 = time.time()
    host = []
    for t in w["t_list"]:
        a = synth.bf16_normal(seed, 0, t, cols)
        b, _, _ = synth.inject_ulp(seed, t, a, frac)
        host.append((a, b))
    a = synth.logit_rows(seed, 0, w["logit_rows"], v)
    b, _, _ = synth.inject_ulp(seed, 99, a, frac)
    host.append((a, b))

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(x).cuda()

    copies = args.copies or COPIES["sweep"]
    sets = [[(dev(a), dev(b)) for a, b in host] for _ in range(copies)]
    torch.cuda.synchronize()
    log(f"[bench] generated and uploaded the sweep ({len(host)} shapes, {copies} copies) in "
        f"{time.time() - t0:.1f}s")
    shape_bytes = [a.size * a.itemsize + b.size * b.itemsize for a, b in host]
    rows_per_step = sum(a.shape[0] for a, _ in host)
    lanes = [torch.cuda.Stream() for _ in range(args.streams)]  # default priority
    outs = [[torch.empty((a.shape[0], L.BITDIFF_ROW_BYTES), dtype=torch.uint8, device="cuda")
             for a, _ in host] for _ in lanes]
    wss = [[torch.empty(int(L.lib().lcmp_bitdiff_workspace_bytes(a.shape[0], a.shape[1])),
                        dtype=torch.uint8, device="cuda") for a, _ in host] for _ in lanes]
    hip = Hip()
    stream = torch.cuda.current_stream()

    def step(i, evs, lane):
        for j, (da, db) in enumerate(sets[i % copies]):
            L.lcmp_bitdiff(da, db, out=outs[lane][j], workspace=wss[lane][j],
                           stream=lanes[lane], events=evs and evs[j])

    # the read-only probe first: its untimed launches settle the clocks
    probe = None
    if not args.no_read_probe:
        probe = read_ceiling(L, [s_[-1] for s_ in sets], hip, torch, stream)
    gpu_ms, wall, per, ev_ms, one_ms = time_steps(step, args.steps, args.warmup, hip, torch,
                                                  stream, lanes, nev=len(host))
    ms_per_step = gpu_ms / args.steps
    kstats = [stats_us(p) for p in per]
    log(f"[bench] {args.steps} sweep steps on {len(lanes)} stream(s): {gpu_ms:.3f} ms; on one "
        f"stream {one_ms:.3f} ms, with timing events {ev_ms:.3f} ms")
    for (a, _), st, nb in zip(host, kstats, shape_bytes):
        log(f"[bench] {list(a.shape)} {a.dtype}: streaming kernel mean {st['mean']:.1f} us, "
            f"median {st['median']:.1f} us, {nb / st['mean'] / 1e3:.1f} GB/s")
    # dominant kernel: the fp32 logit rows (70 % of the bytes)
    big = kstats[-1]
    gbs = lambda nb, us: round(nb / us / 1e3, 1)  # noqa: E731
    achieved = gbs(shape_bytes[-1], big["mean"])
    kern_total_us = sum(st["mean"] for st in kstats)
    roofline = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None, traffic_source=None,
                    kernel="k_row_stats (bitwise only, fp32 [512,151936])",
                    bytes_per_launch=shape_bytes[-1],
                    kernel_us=dict((key, round(val, 1)) for key, val in big.items()),
                    all_kernels_achieved=gbs(sum(shape_bytes), kern_total_us),
                    step_achieved=gbs(sum(shape_bytes), 1e3 * ms_per_step),
                    step_frac=round(gbs(sum(shape_bytes), 1e3 * ms_per_step) / HBM_PEAK_GBS, 4),
                    ms_per_step_one_stream=round(one_ms / args.steps, 4),
                    ms_per_step_timed_pass=round(ev_ms / args.steps, 4))
    if probe is not None:
        roofline["read_ceiling"] = gbs(shape_bytes[-1], probe["median"])
        roofline["frac_of_read_ceiling"] = round(achieved / roofline["read_ceiling"], 4)
        log(f"[bench] read-only probe of the fp32 rows: median {probe['median']:.1f} us")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle_threads()
        # whole sweep steps, repeated until the budget is spent (one step is
        # far below a second of CPU work)
        t1 = time.perf_counter()
        reps = 0
        while reps < 1 or (time.perf_counter() - t1 < args.cpu_seconds and reps < 10000):
            for a, b in host:
                oracle.bitdiff(a, b, nthreads=threads)
            reps += 1
        dt = time.perf_counter() - t1
        cpu = dict(value=reps * rows_per_step / dt, unit="rows/s", cores=threads, kind="oracle",
                   sample=f"{reps} whole sweep steps ({rows_per_step} rows each), {dt:.1f} s",
                   cpu=cpu_model())
        log(f"[bench] cpu oracle: {cpu['value']:.1f} rows/s on {threads} threads")
    value = rows_per_step * args.steps / (gpu_ms / 1e3)
    return {
        "metric": SWEEP_METRIC, "value": round(value, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC["sweep"], "path": "bitdiff",
                   "shapes": [list(a.shape) for a, _ in host],
                   "types": ["bf16" if a.dtype == np.uint16 else "f32" for a, _ in host],
                   "rows_per_step": rows_per_step, "bytes_per_step": sum(shape_bytes),
                   "arithmetic": "integer pattern compares, fp32 differences, fp64 sums",
                   "input_copies": copies, "streams": len(lanes),
                   "hbm_gbs_step": roofline["step_achieved"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="corpus",
                    choices=["corpus", "segment", "stream", "tiny", "sweep"])
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies used in turn (default: 4 for segment and sweep, else 1)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--streams", type=int, default=2,
                    help="streams the value pass spreads consecutive steps over (default 2)")
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
    if args.streams < 1:
        print("bench.py: --streams must be at least 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    import synth
    import logit_distribution_diffing_amd as L

    if args.workload == "sweep":
        rec = run_sweep(args, torch, L, synth)
    else:
        rec = run_compare(args, torch, L, synth)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
