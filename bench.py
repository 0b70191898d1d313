"""Benchmark of the per-token sampler on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload single_stream|window|batch|stress]
python bench.py --summarize-trace KERNEL_STATS_CSV --workload W --cmd "..."
python bench.py --summarize-pmc FETCH_CSV WRITE_CSV --workload W --cmd "..."
python bench.py --summarize-counters COUNTER_CSV... --workload W --cmd "..."
python bench.py --cpu-only     (the oracle's host timing alone)

A step is one pass of the hot path over one batch of the workload:
  single_stream  one row of 248,320 fp32 logits, the sampled chain (top_k 20,
                 top_p 0.8, temperature 0.7) and a greedy pass over the row;
  window         a verify window of 5 rows with penalties over a 64-id history;
  batch          40 rows (8 slots x 5) with per-row parameters and penalties;
  stress         40 bf16-grid rows sampled at top_k 64 with the top-20 raw
                 logprobs of the sampled tokens computed in the same pass, then
                 the logprobs renormalised over 1,000 allowed ids per row.
Logits are resident in HBM before timing.  Each step reads a different copy of
the batch, rotating through at least 512 MiB of copies, so the reads come
from HBM and not from the 256 MiB MALL.  The timed steps are captured once
in a HIP graph and replayed (Philox counters live in device memory and
advance on every call, so replays draw fresh numbers); an eager timing, where
Python launches every call, is reported beside it.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/sec + achieved HBM GB/s (% peak) at V=248,320, top_k=20"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="single_stream",
                    choices=["single_stream", "window", "batch", "stress"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm (same-buffer) figure, so every sampler launch of the run "
                         "reads cold rows (used for the rocprofv3 kernel averages)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads' figures in the JSON line")
    ap.add_argument("--no-alt", action="store_true",
                    help="skip the separate-launch comparison, so every launch of the sampler "
                         "kernel in the run is the step's own (used for the rocprofv3 averages)")
    ap.add_argument("--cpu-reps", type=int, default=10,
                    help="steps per median in the oracle's host timing")
    ap.add_argument("--cpu-only", action="store_true",
                    help="print only the oracle's host timing (no GPU needed)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (known bytes) for counter scaling")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="COUNTER_CSV")
    ap.add_argument("--cmd", default="", help="profiling command recorded in the summary")
    return ap.parse_args()


# ---------------------------------------------------------------- workloads
class Workload:
    """Device-resident copies of one batch plus the prepared calls of one step.
    Philox counters are device-resident and advance on every call, so steps
    captured in a HIP graph draw fresh numbers on every replay."""

    def __init__(self, name, dev):
        import numpy as np
        import torch

        import request_token_sampling_amd as R
        from request_token_sampling_amd import workloads as W

        self.name = name
        hist = hist_len = None
        lp = None
        spec = {}
        self.alt_passes = []
        if name == "single_stream":
            w = W.single_stream()
            x = w["logits"]
            # the sampled and the greedy pass as two parameter rows of one launch
            # over the one logits row (ld = 0); the two-launch form is timed beside
            passes = [("sampled+greedy", w["sampled"] + w["greedy"], 1, 1)]
            self.alt_passes = [("sampled", w["sampled"]), ("greedy", w["greedy"])]
            self.desc = ("single stream: 1 row, V=248,320 fp32 N(0,3) with 3 spiked heads; "
                         "top_k 20, top_p 0.8, min_p 0, temperature 0.7, no penalties; "
                         "plus a greedy pass over the same row (both in one launch)")
        elif name == "window":
            vw = W.VerifyWindows()
            x = vw.next_logits()
            hist = vw.history.reshape(1, -1)
            hist_len = [hist.shape[1]]
            passes = [("sampled", vw.params(0), 5, 5)]
            # argmax drafts (a drafter proposing its own greedy pick per row)
            spec = dict(window=5, draft=torch.from_numpy(
                np.argmax(x, axis=1).astype(np.int32)).to(dev))
            self.desc = ("verify window: 5 rows, V=248,320, penalties 1.1/0.5/0.5 over a "
                         "64-id history, top_k 40, min_p 0.05, top_p 0.95, temperature 1; "
                         "acceptance of argmax drafts in the same launch")
        elif name == "batch":
            w = W.batch_slots()
            x, hist, hist_len = w["logits"], w["history"], w["hist_len"]
            passes = [("sampled", w["params"], 40, 5)]
            self.desc = ("batch slots: 40 rows, V=248,320, per-row T/top_k/top_p/min_p, "
                         "penalties over 256 Zipf history ids per slot")
        else:
            w = W.logprobs_stress()
            x = w["logits"]
            passes = [("sampled+logprobs+allowed", w["params"], 40, 40)]
            ids, off = W.pack_allowed(w["allowed"])
            lp = (w["top_n"], ids, off)
            self.desc = ("logprobs stress: 40 bf16-grid rows, V=248,320, top_k 64, min_p 0.1; "
                         "top-20 raw logprobs of the sampled tokens, and the same renormalised "
                         "over 1,000 allowed ids per row, all in the sampling launch; the "
                         "two-launch form (renormalisation in a second launch) is timed beside")
        self.B, self.V = x.shape
        self.row_bytes = self.V * 4
        batch_bytes = self.B * self.row_bytes
        self.ncopies = max(2, math.ceil(ROTATE_BYTES / batch_bytes))
        base = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.copies = base.unsqueeze(0).repeat(self.ncopies, 1, 1)
        self.hist = None if hist is None else torch.from_numpy(np.asarray(hist, np.int32)).to(dev)
        self.hist_len = hist_len
        self.first_params = self.alt_passes[0][1] if self.alt_passes else passes[0][1]
        self.ws = R.make_workspace(max([self.B] + [len(p[1]) for p in passes]), self.V, dev)
        self.calls, self.labels = [], []
        self.sampled_rows = 0
        lp_ids = None if lp is None else torch.from_numpy(lp[1]).to(dev)
        if lp is not None:
            spec = dict(spec, logprob_allowed=lp_ids, logprob_allowed_off=lp[2])
        for label, params, counted, stride in passes:
            ctr = torch.tensor([p.get("counter", 0) for p in params], dtype=torch.int64,
                               device=dev)
            self.calls.append(R.SampleCall(self.view(self.copies[0], len(params)), params,
                                           self.hist, hist_len, workspace=self.ws, counters=ctr,
                                           counter_stride=stride,
                                           logprobs=None if lp is None else lp[0], **spec))
            self.labels.append(label)
            self.sampled_rows += counted
        self.param_rows = sum(c.B for c in self.calls)
        self.alt_calls = [R.SampleCall(self.copies[0], params, self.hist, hist_len,
                                       workspace=self.ws) for _, params in self.alt_passes]
        self.alt_labels = [l for l, _ in self.alt_passes]
        # bytes a step moves besides the logit rows and the sampling outputs:
        # logprob outputs, and the allowed lists with the logits they gather
        self.extra_bytes = 0
        if lp is not None:
            top_n, ids, off = lp
            self.extra_bytes = 2 * self.param_rows * (4 + 8 * top_n) + 8 * int(ids.size)
            # the two-launch form: sampling with raw logprobs, then the
            # allowed-id logprob kernels on the sampled tokens
            ctr = torch.tensor([p.get("counter", 0) for p in passes[0][1]], dtype=torch.int64,
                               device=dev)
            first = R.SampleCall(self.copies[0], passes[0][1], workspace=self.ws, counters=ctr,
                                 counter_stride=passes[0][3], logprobs=top_n)
            self.alt_calls = [first, R.LogprobCall(self.copies[0], first.token, top_n, lp_ids,
                                                   off, workspace=self.ws)]
            self.alt_labels = ["sampled+logprobs", "logprobs_allowed"]
        self.passes = list(self.labels)
        self.torch = torch

    @staticmethod
    def view(x, rows):
        """The logits as `rows` parameter rows: the batch itself, or its one
        row broadcast (ld = 0) when several parameter rows share it."""
        return x if rows == x.shape[0] else x.expand(rows, -1)

    def step(self, i):
        x = self.copies[i % self.ncopies]
        for c in self.calls:
            c.logits = self.view(x, c.B)
            c()


def time_eager(wl, steps, warmup):
    """Wall time of `steps` eager steps (Python launches each call)."""
    torch = wl.torch
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(warmup + i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_graph(wl, steps, warm=False):
    """Wall time of `steps` steps replayed from one captured HIP graph.  With
    `warm` every step reads the same logits copy, so the rows come from the
    caches instead of HBM (context for the cold figure, never the value)."""
    torch = wl.torch
    wl.step(0)                      # eager warm-up of every kernel variant
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            wl.step(0 if warm else i)
    torch.cuda.synchronize()
    graph.replay()                  # warm-up replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    return wall


def kernel_durations(wl, steps):
    """Average duration of each sampler call from two HIP events on its launch
    stream around `steps` back-to-back launches of that call alone (rotating
    logit copies).  The stream is first held by a sleep kernel so the host
    enqueues ahead: the events then bracket the kernels and the dispatch gaps
    between them, not the host's launch latency."""
    torch = wl.torch
    out = []
    for c in wl.calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(steps * 0.05e-3 * 2.0e9))
        e0.record()
        for i in range(steps):
            c.logits = wl.view(wl.copies[i % wl.ncopies], c.B)
            c()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def roofline(wl, kern_ms):
    """HBM roofline of the sampler kernel: algorithmic bytes per launch (one
    read of every logit row, plus outputs) over its average launch duration
    (all sampler launches of a step: they are one kernel)."""
    out_bytes = wl.param_rows * (4 + 12 + 256 + 256 + 4 + 8) + wl.extra_bytes
    alg = wl.B * wl.row_bytes + out_bytes
    avg_ms = sum(kern_ms) / len(kern_ms)
    achieved = alg / (avg_ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=read_traffic(wl.name),
                kernel="rts::sample_kernel", algorithmic_bytes_per_launch=alg,
                avg_launch_us=round(avg_ms * 1e3, 3),
                per_call_us={l: round(m * 1e3, 3) for l, m in zip(wl.labels, kern_ms)})


def read_floor(wl, launches=400):
    """The practical bandwidth floor beside the roofline: rts_read_rows (the
    sampler's grid, chunking and loads with only a chunk maximum) over the
    same rotating copies, replayed from a captured graph; per-launch time."""
    import request_token_sampling_amd as R
    torch = wl.torch
    rc = R.ReadCall(wl.copies[0])

    def launch(i):
        rc.logits = wl.copies[i % wl.ncopies]
        rc()

    launch(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(launches):
            launch(i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / launches * 1e6
    del graph
    gbs = wl.B * wl.row_bytes / (us * 1e-6) / 1e9
    return dict(kernel="rts::read_rows_kernel", us_per_launch=round(us, 3), achieved=round(gbs, 1),
                frac=round(gbs / HBM_PEAK_GBS, 4))


def per_launch_us(wl, call, launches):
    """Average time of `launches` back-to-back launches of one prepared call
    over rotating copies, between two events with the host enqueued ahead."""
    torch = wl.torch
    call.logits = wl.view(wl.copies[0], call.B)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(launches * 0.05e-3 * 2.0e9))
    e0.record()
    for i in range(launches):
        call.logits = wl.view(wl.copies[i % wl.ncopies], call.B)
        call()
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) / launches * 1e3, 2)


def ablations(dev):
    """The pages' earlier designs (one thread per row with k rescans; one
    workgroup per row with k argmax rounds and a penalty bitmap; the same with
    the per-candidate recount) against the single-pass kernel, same outputs,
    microseconds per launch."""
    import request_token_sampling_amd as R
    out = {}
    for name, launches in (("single_stream", 8), ("window", 4)):
        wl = Workload(name, dev)
        params = wl.first_params
        ws = R.make_workspace(wl.B, wl.V, dev)
        single = R.SampleCall(wl.copies[0], params, wl.hist, wl.hist_len, workspace=ws)
        res = {"single_pass_us": per_launch_us(wl, single, 300)}
        if name == "single_stream":
            # the greedy pass alone (top_k 1): selection, merge and epilogue
            # at their shortest, over the same row
            greedy = R.SampleCall(wl.copies[0], wl.alt_passes[1][1], workspace=ws)
            res["greedy_only_us"] = per_launch_us(wl, greedy, 300)
        for label, design, n in (("prior_block_us", R.PRIOR_BLOCK, 4 * launches),
                                 ("prior_recount_us", R.PRIOR_RECOUNT, launches),
                                 ("prior_thread_us", R.PRIOR_THREAD, launches)):
            call = R.PriorCall(design, wl.copies[0], params, wl.hist, wl.hist_len, workspace=ws)
            res[label] = per_launch_us(wl, call, n)
            progress(f"ablation {name}: {label} {res[label]} us")
        res["rows"] = wl.B
        out[name] = res
        del wl
        wl = None
        import torch
        torch.cuda.empty_cache()
    return out


def time_alt_graph(wl, steps):
    """Per-step wall time with the passes of a step as separate launches
    (single stream: the sampled pass, then the greedy pass; stress: sampling
    with raw logprobs, then the allowed-id logprob pass), graph-replayed."""
    torch = wl.torch
    for c in wl.alt_calls:
        c()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            for c in wl.alt_calls:
                c.logits = wl.copies[i % wl.ncopies]
                c()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    return wall / steps


def measure(wl, steps, warmup, warm=True, alt=True):
    eager = time_eager(wl, steps, warmup)
    graph = time_graph(wl, steps)
    warm = time_graph(wl, steps, warm=True) if warm else None
    # at least 300 launches whatever K is: a short run's first launches run slow
    kern = kernel_durations(wl, max(300, min(steps, 500)))
    alt = time_alt_graph(wl, steps) if (alt and wl.alt_calls) else None
    return dict(graph_wall=graph, warm_wall=warm, eager_wall=eager, kern_ms=kern,
                floor=read_floor(wl), alt=alt)


def read_traffic(workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"traffic_sample_kernel_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# The sources rts::sample_kernel is compiled from: the counters in profiles/
# describe that kernel, so only a change to these makes them stale.
SAMPLE_KERNEL_SOURCES = ("rts_sample.hip", "rts_epilogue.h", "rts_renorm.h", "rts_select.h",
                         "rts_device.h", "rts_internal.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "request_token_sampling_amd", "csrc")
    for f in SAMPLE_KERNEL_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


COPY_BYTES = 256 << 20


def calibration_copy(dev):
    """A plain device-to-device copy of COPY_BYTES, three times: the HBM
    counters of these dispatches calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(path, workload, cmd):
    """Text summary of a rocprofv3 --kernel-trace --stats kernel_stats.csv."""
    rows = _csv_rows(path)
    lines = [f"# rocprofv3 kernel statistics, workload {workload}",
             f"# command: {cmd}",
             f"# summarised by: python bench.py --summarize-trace {os.path.basename(path)} "
             f"--workload {workload}",
             "kernel | calls | average_us | min_us | max_us | percent"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or ""
        if not name:
            continue
        def us(key):
            v = r.get(key)
            return f"{float(v) / 1000:.3f}" if v not in (None, "") else "-"
        lines.append(f"{name[:90]} | {r.get('Calls', '-')} | {us('AverageNs')} | {us('MinNs')} | "
                     f"{us('MaxNs')} | {float(r.get('Percentage', 0)):.2f}")
    out = os.path.join(PROFILES, f"sample_kernel_{workload}.txt")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


# logit bytes one launch of each workload reads (rows x V x 4)
WORKLOAD_LOGIT_BYTES = {"single_stream": 1 * 248320 * 4, "window": 5 * 248320 * 4,
                        "batch": 40 * 248320 * 4, "stress": 40 * 248320 * 4}


def summarize_counters(paths, workload, cmd):
    """Median per sampler dispatch of every counter in one or more rocprofv3
    --pmc counter_collection.csv files (one pass each), with ratios that say
    where the waves' cycles go."""
    import statistics
    vals = {}
    for path in paths:
        for r in _csv_rows(path):
            if "rts::sample_kernel" not in r.get("Kernel_Name", ""):
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in sorted(vals.items())}
    lines = [f"# rocprofv3 counters of rts::sample_kernel, workload {workload}: median per "
             f"dispatch over all sampler dispatches",
             f"# command (one pass per counter group): {cmd}",
             "# summarised by: python bench.py --summarize-counters "
             + " ".join(os.path.basename(p) for p in paths) + f" --workload {workload}"]
    for k, v in med.items():
        lines.append(f"{k} = {v:.1f}")
        lines.append(f"{k}_dispatches = {len(vals[k])}")

    def ratio(name, a, b):
        if a in med and b in med and med[b] > 0:
            lines.append(f"{name} = {med[a] / med[b]:.4f}")
    ratio("wait_any_per_wave_cycle", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")
    ratio("valu_active_per_wave_cycle", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")
    ratio("salu_per_valu_inst", "SQ_INSTS_SALU", "SQ_INSTS_VALU")
    ratio("lds_per_valu_inst", "SQ_INSTS_LDS", "SQ_INSTS_VALU")
    ratio("wait_any_per_wave_cycle_all", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
    ratio("lds_bank_conflict_per_lds_active", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")
    if "SQ_WAVES" in med and med["SQ_WAVES"] > 0:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_SMEM",
                  "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_WAVE_CYCLES"):
            if k in med:
                lines.append(f"{k}_per_wave = {med[k] / med['SQ_WAVES']:.1f}")
    lines.append(f"source_sha256 = {kernel_source_hash()}")
    out = os.path.join(PROFILES, f"counters_sample_kernel_{workload}.txt")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(fetch_csv, write_csv, workload, cmd):
    """HBM bytes per sampler launch from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the calibration copy of COPY_BYTES."""
    import statistics

    def per_kernel(path, counter):
        """Counter values of the sampler dispatches, and of the first three
        copy dispatches of the run: the calibration copies, which run before
        anything else copies on the device."""
        sample, copies, reads = [], [], []
        for r in _csv_rows(path):
            if r.get("Counter_Name") != counter:
                continue
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            if "rts::sample_kernel" in name:
                sample.append(val)
            elif "read_rows_kernel" in name:
                reads.append(val)
            elif "copy" in name.lower():
                copies.append((int(r["Dispatch_Id"]), val))
        copies.sort()
        return {"sample": sample, "copy": [v for _, v in copies[:3]], "read": reads}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    f_copy, w_copy = statistics.median(f["copy"]), statistics.median(w["copy"])
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    f_s, w_s = statistics.median(f["sample"]), statistics.median(w["sample"])
    fetch_b, write_b = f_s * 1024.0 * f_scale, w_s * 1024.0 * w_scale
    lines = [f"# HBM traffic of rts::sample_kernel, workload {workload}",
             f"# command (FETCH_SIZE pass, then WRITE_SIZE pass): {cmd}",
             f"# summarised by: python bench.py --summarize-pmc {os.path.basename(fetch_csv)} "
             f"{os.path.basename(write_csv)} --workload {workload}",
             f"# calibration: a {COPY_BYTES} B device copy reads FETCH_SIZE {f_copy:.1f} KiB and "
             f"writes WRITE_SIZE {w_copy:.1f} KiB per dispatch",
             f"fetch_scale = {f_scale:.4f}",
             f"write_scale = {w_scale:.4f}",
             f"sample_dispatches = {len(f['sample'])}",
             f"fetch_kib_per_launch_raw = {f_s:.1f}",
             f"write_kib_per_launch_raw = {w_s:.1f}",
             f"fetch_bytes_per_launch = {fetch_b:.0f}",
             f"write_bytes_per_launch = {write_b:.0f}",
             f"hbm_bytes_per_launch = {fetch_b + write_b:.0f}",
             f"source_sha256 = {kernel_source_hash()}"]
    if f["read"]:
        # second calibration: rts_read_rows reads every logit of the batch
        # once with the sampler's own loads, a known byte count per launch
        known = WORKLOAD_LOGIT_BYTES[workload]
        r_kib = statistics.median(f["read"])
        lines += [f"read_rows_dispatches = {len(f['read'])}",
                  f"read_rows_fetch_kib_raw = {r_kib:.1f}",
                  f"read_rows_known_bytes = {known}",
                  f"read_rows_fetch_scale = {known / (r_kib * 1024.0):.4f}",
                  f"fetch_bytes_per_launch_read_rows_scale = "
                  f"{f_s * 1024.0 * known / (r_kib * 1024.0):.0f}"]
    out = os.path.join(PROFILES, f"traffic_sample_kernel_{workload}.txt")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def host_threads():
    """Host cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _oracle_step(name):
    """One workload's step as oracle calls, one job per row: (jobs, rows
    counted, logit bytes read).  Each job is independent of the others."""
    import oracle.oracle as O
    from request_token_sampling_amd import workloads as W

    if name == "tiny":
        w = W.tiny()
        x = w["logits"]
        jobs = [lambda r=r, p=p: O.sample_row(x[r], p)
                for ps in (w["sampled"], w["greedy"]) for r, p in enumerate(ps)]
        return jobs, x.shape[0], x.nbytes, "4 rows of V=1,024, sampled and greedy passes"
    if name == "single_stream":
        w = W.single_stream()
        x = w["logits"][0]
        jobs = [lambda p=p: O.sample_row(x, p) for p in w["sampled"] + w["greedy"]]
        return jobs, 1, x.nbytes, "one sampled row of V=248,320 and its greedy pass"
    if name == "window":
        vw = W.VerifyWindows()
        x = vw.next_logits()
        hist = vw.history.reshape(-1)
        jobs = [lambda r=r: O.sample_row(x[r], p, hist) for r, p in enumerate(vw.params(0))]
        return jobs, x.shape[0], x.nbytes, "a verify window of 5 penalised rows"
    if name == "batch":
        w = W.batch_slots()
        x, h, hl = w["logits"], w["history"], w["hist_len"]

        def row(r, p):
            hr = p.get("history_row", -1)
            return O.sample_row(x[r], p, None if hr < 0 else h[hr][:int(hl[hr])])
        jobs = [lambda r=r, p=p: row(r, p) for r, p in enumerate(w["params"])]
        return jobs, x.shape[0], x.nbytes, "40 penalised batch-slot rows"
    w = W.logprobs_stress()
    x, top_n = w["logits"], w["top_n"]

    def row(r, p):
        t = O.sample_row(x[r], p)["token"]
        O.token_logprobs_row(x[r], t, top_n)
        return O.token_logprobs_row(x[r], t, top_n, w["allowed"][r])
    jobs = [lambda r=r, p=p: row(r, p) for r, p in enumerate(w["params"])]
    return jobs, x.shape[0], x.nbytes, ("40 rows sampled at top_k 64 with top-20 raw logprobs "
                                        "and the same over 1,000 allowed ids")


def cpu_baseline(reps=10):
    """The oracle (its C source built -O3 -march=native, same arithmetic as
    the tests' build) on the host: for each workload, the median of `reps`
    steps, once on one thread and once with rows spread over every host core
    (one row per job; the C calls release the GIL).  The one-thread leg of
    the 40-row workloads times the first 10 rows of the batch (rows/s is per
    row).  `value` is the single-stream step on every core."""
    import statistics
    from concurrent.futures import ThreadPoolExecutor

    import oracle.oracle as O
    O.use_native_build()
    cores = host_threads()
    out = {}
    try:
        for name in ("tiny", "single_stream", "window", "batch", "stress"):
            jobs, rows, nbytes, what = _oracle_step(name)
            res = {"sample": what}
            for threads in (1, cores):
                part = jobs[:10] if threads == 1 and len(jobs) > 10 else jobs
                frac = len(part) / len(jobs)
                times = []
                with ThreadPoolExecutor(max_workers=threads) as ex:
                    for _ in range(reps):
                        t0 = time.perf_counter()
                        list(ex.map(lambda f: f(), part))
                        times.append(time.perf_counter() - t0)
                t = statistics.median(times)
                res[f"threads_{threads}"] = dict(
                    threads=min(threads, len(part)), cores=cores, reps=reps,
                    jobs_per_rep=len(part), median_s=round(t, 5),
                    rows_s=round(rows * frac / t, 3), gb_s=round(nbytes * frac / t / 1e9, 4))
                progress(f"oracle {name}: {threads} thread(s) {t * 1e3:.1f} ms per rep")
            out[name] = res
    finally:
        O.use_native_build(False)
    top = out["single_stream"][f"threads_{cores}"]
    return dict(value=top["rows_s"], unit="rows/s", cores=top["threads"], kind="oracle",
                host_cores=cores, build="gcc -O3 -march=native -ffp-contract=off",
                sample=(f"median of {reps} single-stream steps (one sampled row of V=248,320 "
                        f"and its greedy pass, one job each) over {top['threads']} host "
                        f"threads; every workload at 1 thread and at {cores} in by_workload"),
                by_workload=out)


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.cmd)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.cmd)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.cmd)
        return
    if args.cpu_only:
        print(json.dumps(cpu_baseline(args.cpu_reps)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the sampler's rows are independent, so a batch "
              "shards by rows with no exchange and one GPU's share is the measured unit; run it "
              "with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    if args.calibration_copy:
        calibration_copy(dev)
    wl = Workload(args.workload, dev)
    progress(f"{args.workload}: {wl.ncopies} copies resident, timing {args.steps} steps")
    m = measure(wl, args.steps, args.warmup, warm=not args.no_warm, alt=not args.no_alt)
    progress(f"{args.workload}: graph {m['graph_wall'] / args.steps * 1e3:.4f} ms/step, eager "
             f"{m['eager_wall'] / args.steps * 1e3:.4f} ms/step, kernels {m['kern_ms']}")
    value = wl.sampled_rows * args.steps / m["graph_wall"]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["graph_wall"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.desc, "rows_per_step": wl.B, "V": wl.V,
                   "passes_per_step": wl.passes, "launch": "hip_graph_replay",
                   "philox_counters": "device-resident, advanced per call",
                   "logit_copies_rotated": wl.ncopies, "device": props.name},
        "roofline": dict(roofline(wl, m["kern_ms"]), read_floor=m["floor"]),
        "eager": {"value": round(wl.sampled_rows * args.steps / m["eager_wall"], 1),
                  "ms_per_step": round(m["eager_wall"] / args.steps * 1e3, 5)},
    }
    if m["warm_wall"] is not None:
        line["warm"] = {"value": round(wl.sampled_rows * args.steps / m["warm_wall"], 1),
                        "ms_per_step": round(m["warm_wall"] / args.steps * 1e3, 5),
                        "note": "every step reads the same logits copy (cache-resident); "
                                "context only"}
    if m["alt"] is not None:
        line["separate_launches"] = {"value": round(wl.sampled_rows / m["alt"], 1),
                                     "ms_per_step": round(m["alt"] * 1e3, 5),
                                     "passes": wl.alt_labels}
    if not args.no_extra:
        extra = {}
        for name in ("batch", "stress", "window"):
            if name == args.workload:
                continue
            w2 = Workload(name, dev)
            steps = max(300, args.steps // 4)
            m2 = measure(w2, steps, max(10, args.warmup // 4), warm=not args.no_warm,
                         alt=not args.no_alt)
            progress(f"{name}: graph {m2['graph_wall'] / steps * 1e3:.4f} ms/step, kernels "
                     f"{m2['kern_ms']}")
            extra[name] = dict(value=round(w2.sampled_rows * steps / m2["graph_wall"], 1),
                               unit="rows/s", steps=steps,
                               ms_per_step=round(m2["graph_wall"] / steps * 1e3, 5),
                               eager_ms_per_step=round(m2["eager_wall"] / steps * 1e3, 5),
                               warm_ms_per_step=(None if m2["warm_wall"] is None
                                                 else round(m2["warm_wall"] / steps * 1e3, 5)),
                               roofline=dict(roofline(w2, m2["kern_ms"]), read_floor=m2["floor"]),
                               desc=w2.desc,
                               passes_per_step=w2.passes)
            if m2["alt"] is not None:
                extra[name]["separate_launches"] = dict(ms_per_step=round(m2["alt"] * 1e3, 5),
                                                        passes=w2.alt_labels)
            del w2
            torch.cuda.empty_cache()
        line["other_workloads"] = extra
    if not args.no_extra:
        line["ablations"] = ablations(dev)
    if not args.no_cpu_baseline:
        progress("oracle on the host: every workload, 1 thread and all host cores")
        line["cpu_baseline"] = cpu_baseline(args.cpu_reps)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
