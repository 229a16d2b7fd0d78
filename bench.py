#!/usr/bin/env python3
"""Benchmark of the MI355X decode-attention library.

One step is one pass of the whole decode-attention hot path over one batch of
synthetic input: a slidingDecodeGQA call on the contiguous bf16 cache of
B=256 sequences (S_max 8192, seq_lens uniform in [1, 8192], window 1024) and a
decodeGQA call on the paged bf16 cache of B=32 sequences (seq_lens uniform in
[16384, 131072], page 16, random page permutation) -- the split kernels, the
split-S combine and the paged addressing all run every step.  Inputs are
resident in HBM before timing starts.

Prints one JSON line: value = algorithmic K/V bytes of the step / step time
(GB/s), with per-kernel launch durations taken from HIP events the library
records on its launch stream during the timed region, the roofline of the
dominant kernel against the 8 TB/s HBM3E peak (beside the figure the committed
rocprofv3 trace gives), every other workload of the shape domain timed as
single calls after a cache-evicting read, the widened calls (runtime window,
capped cache, keys from values, append, prefill), and the fp64 CPU oracle
timed on the step's workload.

--only SECTION[,SECTION...] runs a subset (for one profiler pass per
workload); --summarize-trace turns a rocprofv3 kernel trace of such a run
into per-kernel figures.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import socket
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = ("decode-attn K/V read GB/s and % of HBM peak; µs per call "
          "(sliding B=256, global B=32)")
SLIDING = "sliding_bf16_b256_s8192"
GLOBAL = "global_bf16_b32_paged_s16k_128k"
SMALL = ("sliding_f32_b4_s2048", "global_bf16_b4_s4096")
LONG = ("global_bf16_b1_paged_s262144", "sliding_bf16_b1_paged_s262144")
# runtime windows of the sliding geometry measured beside the step (per-layer
# windows of the Retrofit Plan page's progressive window table)
SWEEP_WINDOWS = (2048, 4096, 8192)
SECTIONS = ("step", "small", "window", "append", "kfv", "ring", "long", "prefill", "probe")
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "hbm_traffic_sliding_b256_global_b32_paged.txt")
TRACE_FILE = os.path.join(PROFILES, "kernel_trace_sliding_b256_global_b32_paged.txt")
# the sources of the decode and append kernels (the profiled ones)
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_slidingdecodegqa_amd", "csrc", f)
                  for f in ("gqa_common.h", "gqa_decode.hip")]
# untimed calls before each timed section after the step: the first calls
# after a switch of workload run measurably slower
SECTION_WARMUP = 10
FLUSH_BYTES = 2 << 30   # a read of this many bytes evicts L2 and the 256 MB MALL
SINGLE_CALLS = 50       # flushed single calls per workload (median reported)
CPU_SHARE = 16          # host threads allotted to one GPU on the measuring machine


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--only", type=str, default=",".join(SECTIONS),
                    help="comma-separated sections to run: " + ",".join(SECTIONS))
    ap.add_argument("--single-calls", type=int, default=SINGLE_CALLS,
                    help="flushed single calls per workload (median reported)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (e.g. under a profiler)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run the library's plain read stream and plain copy over BYTES "
                         "bytes (calibrates a profiler's HBM byte counters) and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the prefill workloads (one JSON line) and exit")
    ap.add_argument("--summarize-trace", type=str, default=None, metavar="CSV",
                    help="summarise a rocprofv3 kernel_trace.csv (per kernel: all launches, and "
                         "the launches after the first --skip of each kernel) and exit")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --summarize-trace: leading launches of each kernel to leave out")
    ap.add_argument("--take", type=int, default=0,
                    help="with --summarize-trace: launches to keep after the skipped ones "
                         "(0: all)")
    return ap.parse_args()


# ------------------------------------------------------------ measurement aids

def source_hash() -> str:
    """sha256 over the decode kernels' sources, in order."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_keyed(path):
    """key = value lines of a committed profile summary (comments dropped)."""
    vals = {}
    if not os.path.exists(path):
        return vals
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = v
    return vals


def read_traffic(key: str = "global_main"):
    """HBM bytes per launch of a kernel (global_main: the dominant kernel) from
    committed rocprofv3 --pmc runs, valid only if taken on the current kernel
    source."""
    vals = read_keyed(TRAFFIC_FILE)
    if vals.get("source_sha256") != source_hash():
        return None
    try:
        return float(vals[f"{key}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_trace(key: str = "global_main"):
    """(average timed launch in us, box, source matches) of a kernel in the
    committed kernel trace of the bench step."""
    vals = read_keyed(TRACE_FILE)
    try:
        us = float(vals[f"{key}_avg_us_timed"])
    except (KeyError, ValueError):
        return None, None, False
    return us, vals.get("box"), vals.get("source_sha256") == source_hash()


def box_name() -> str:
    """The machine: host name and the device's UUID (PCI bus id without one)."""
    try:
        import torch
        props = torch.cuda.get_device_properties(0)
        dev = str(getattr(props, "uuid", "") or "") or f"pci{getattr(props, 'pci_bus_id', '?')}"
    except Exception:  # pragma: no cover - measurement metadata only
        dev = "?"
    return f"{socket.gethostname()}/{dev}"


def summarize_trace(path: str, skip: int, take: int = 0) -> dict:
    """Per kernel of a rocprofv3 kernel_trace.csv: launches and durations, over
    all launches and over the `take` launches (0: all) after the first `skip`
    of each kernel (the timed steps of a run with --warmup skip --steps take)."""
    per = {}
    for r in csv.DictReader(open(path)):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), d))
    out = {}
    for name, lst in per.items():
        lst.sort()
        d_all = [x[1] for x in lst]
        d_t = d_all[skip:skip + take] if take > 0 else d_all[skip:]
        d_t = d_t or d_all
        out[name] = {"calls": len(d_all), "avg_us": round(statistics.fmean(d_all), 2),
                     "calls_after_skip": len(d_t), "avg_us_after_skip": round(statistics.fmean(d_t), 2),
                     "median_us_after_skip": round(statistics.median(d_t), 2),
                     "min_us": round(min(d_all), 2), "max_us": round(max(d_all), 2)}
    return out


def hbm_probes(nbytes: int, reps: int = 3) -> dict:
    """The library's plain read stream and plain copy over nbytes of random data."""
    import torch
    import decode_attention_slidingdecodegqa_amd as gqa
    n = nbytes // 4
    g = torch.Generator(device="cuda").manual_seed(1)
    src = torch.rand(n, dtype=torch.float32, device="cuda", generator=g)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = {"probe_bytes": n * 4}
    for name, fn, moved in (("read", lambda: gqa.hbm_read_probe(src, sink), n * 4),
                            ("copy", lambda: gqa.hbm_copy_probe(src, dst), 2 * n * 4)):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        out[f"{name}_ms"] = round(best, 4)
        out[f"{name}_GBps"] = round(moved / (best * 1e-3) / 1e9, 1)
    return out


def frac(nbytes, us):
    return round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if us else None


def gbps(nbytes, us):
    return round(nbytes / (us * 1e-6) / 1e9, 1) if us else None


class Timer:
    """Call timing on one stream: back-to-back mean, and the median of flushed
    single calls (each after a read of FLUSH_BYTES that evicts the caches; a
    read leaves no dirty lines for the call to write back)."""

    def __init__(self, stream, dev):
        import torch
        self.torch = torch
        self.stream = stream
        self.dev = dev
        self.flush_buf = None

    def _ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def warm(self, call, reps):
        a, b = self._ev(), self._ev()
        a.record(self.stream)
        for _ in range(reps):
            call()
        b.record(self.stream)
        self.torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    def single(self, call, n, flush=True):
        torch = self.torch
        if flush and self.flush_buf is None:
            self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=self.dev)
        a, b = self._ev(), self._ev()
        t = []
        for _ in range(n):
            if flush:
                self.flush_buf.sum()
            torch.cuda.synchronize()
            a.record(self.stream)
            call()
            b.record(self.stream)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) * 1e3)
        return statistics.median(t)

    def queued(self, call, n):
        """Median of n flushed single calls, each queued behind its flush with
        no host synchronisation in between: the call's launch (host) cost is
        hidden behind the flush, as behind the previous layer's work in a
        decode step, so the span is the call's own device latency with cold
        caches."""
        torch = self.torch
        if self.flush_buf is None:
            self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=self.dev)
        t = []
        for _ in range(n):
            a, b = self._ev(), self._ev()
            self.flush_buf.sum()
            a.record(self.stream)
            call()
            b.record(self.stream)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) * 1e3)
        return statistics.median(t)

    def graph(self, call, reps):
        """Mean per call of `reps` back-to-back calls replayed from one HIP
        graph (captured once, replayed three times, the last two timed): the
        device time per call with no host launch cost in the loop."""
        torch = self.torch
        side = torch.cuda.Stream(self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream(self.dev).wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                call()
        g.replay()
        torch.cuda.synchronize()
        a, b = self._ev(), self._ev()
        a.record(self.stream)
        g.replay()
        g.replay()
        b.record(self.stream)
        torch.cuda.synchronize()
        del g
        us = a.elapsed_time(b) / (2 * reps) * 1e3
        if us < 1.0:  # a call launched outside the capture stream ran eagerly
            raise RuntimeError(f"the captured graph holds no decode work ({us:.2f} us per call)")
        return us

    def release(self):
        self.flush_buf = None


def kernel_us(prof, variant):
    """Mean main and combine kernel durations (us) from the library's events."""
    def avg(key):
        n, t = prof[key]
        return t / n * 1e3 if n else 0.0
    return avg((variant, "main")), avg((variant, "combine"))


# ------------------------------------------------------------------ sections

class Ctx:
    def __init__(self, args):
        import torch
        import decode_attention_slidingdecodegqa_amd as gqa
        import synth
        self.args, self.torch, self.gqa, self.synth = args, torch, gqa, synth
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream(self.dev)
        self.timer = Timer(self.stream, self.dev)
        self._sl = self._gl = None

    def sl(self):
        if self._sl is None:
            log("generating the sliding B=256 contiguous cache (rows drawn for the widest window)")
            self._sl = self.synth.make_workload(SLIDING, seed=self.args.seed, device=self.dev,
                                                fill=0.0, window=max(SWEEP_WINDOWS))
        return self._sl

    def gl(self):
        if self._gl is None:
            log("generating the global B=32 paged cache")
            self._gl = self.synth.make_workload(GLOBAL, seed=self.args.seed, device=self.dev,
                                                fill=0.0)
        return self._gl

    def workspace(self, variant, B, cap, window=None):
        need = self.gqa.gqa_decode_workspace_bytes(variant, B, cap, window)
        return self.torch.empty(max(need, 256), dtype=self.torch.uint8, device=self.dev)

    def decode_call(self, c, o, ws, window=None):
        """The call on the current stream (self.stream outside a graph capture,
        the capture stream inside one)."""
        gqa = self.gqa
        if window is not None:
            if c.block_table is None:
                return lambda: gqa.gqa_decode_sliding_window(c.q, c.k, c.v, c.seq_lens, window,
                                                             o=o, workspace=ws,
                                                             stream=None)
            return lambda: gqa.gqa_decode_sliding_window_paged(c.q, c.k, c.v, c.block_table,
                                                               c.seq_lens, window, o=o,
                                                               workspace=ws, stream=None)
        fn = {("sliding", False): gqa.gqa_decode_sliding, ("global", False): gqa.gqa_decode_global,
              ("sliding", True): gqa.gqa_decode_sliding_paged,
              ("global", True): gqa.gqa_decode_global_paged}[(c.variant, c.paged)]
        if c.paged:
            return lambda: fn(c.q, c.k, c.v, c.block_table, c.seq_lens, o=o, workspace=ws,
                              stream=None)
        return lambda: fn(c.q, c.k, c.v, c.seq_lens, o=o, workspace=ws, stream=None)


def section_step(ctx, line):
    """The graded step (sliding B=256 + global B=32 paged): the headline value
    and the roofline of the dominant kernel."""
    args, torch, gqa = ctx.args, ctx.torch, ctx.gqa
    sl, gl = ctx.sl(), ctx.gl()
    sl_bytes, gl_bytes = sl.kv_bytes(window=1024), gl.kv_bytes()
    o_sl, o_gl = torch.empty_like(sl.q), torch.empty_like(gl.q)
    ws_sl = ctx.workspace("sliding", sl.B, sl.cap)
    ws_gl = ctx.workspace("global", gl.B, gl.cap)
    call_sl = ctx.decode_call(sl, o_sl, ws_sl)
    call_gl = ctx.decode_call(gl, o_gl, ws_gl)

    def step():
        call_sl()
        call_gl()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warm-up done ({args.warmup} steps)")
    gqa.profile_begin(4 * args.steps + 8)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(ctx.stream)
    for _ in range(args.steps):
        step()
    stop.record(ctx.stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    prof = gqa.profile_read()
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step")
    sl_main, sl_comb = kernel_us(prof, "sliding")
    gl_main, gl_comb = kernel_us(prof, "global")
    sl_us, gl_us = sl_main + sl_comb, gl_main + gl_comb
    line["value"] = round((sl_bytes + gl_bytes) / (ms_step * 1e-3) / 1e9, 1)
    line["ms_per_step"] = round(ms_step, 4)
    cfg = line["config"]
    cfg["sliding"] = {
        "B": sl.B, "S_max": sl.cap, "kv_heads": 16, "head_dim": 256, "window": 1024,
        "cache": "contiguous", "kv_bytes_per_call": sl_bytes, "us_per_call": round(sl_us, 2),
        "main_kernel_us": round(sl_main, 2), "combine_kernel_us": round(sl_comb, 2),
        "kv_GBps": gbps(sl_bytes, sl_us), "frac_of_hbm_peak": frac(sl_bytes, sl_us),
        "plan": gqa.gqa_decode_plan("sliding", sl.B, sl.cap)}
    cfg["global"] = {
        "B": gl.B, "max_pages": gl.block_table.shape[1], "num_pages": gl.k.shape[0],
        "kv_heads": 4, "head_dim": 512, "cache": "paged16", "kv_bytes_per_call": gl_bytes,
        "us_per_call": round(gl_us, 2), "main_kernel_us": round(gl_main, 2),
        "combine_kernel_us": round(gl_comb, 2), "kv_GBps": gbps(gl_bytes, gl_us),
        "frac_of_hbm_peak": frac(gl_bytes, gl_us),
        "plan": gqa.gqa_decode_plan("global", gl.B, gl.cap)}
    # each call also timed on its own (events around one call, the stream
    # drained in between): the median of 50 (their read sets exceed the caches)
    for name, call, nb in (("sliding", call_sl, sl_bytes), ("global", call_gl, gl_bytes)):
        med = ctx.timer.single(call, 50, flush=False)
        cfg[name]["us_per_call_median_of_50_single"] = round(med, 2)
        cfg[name]["frac_of_hbm_peak_median_single"] = frac(nb, med)
    cfg["c2_sliding_b256_us"] = cfg["sliding"]["us_per_call_median_of_50_single"]
    cfg["c2_sliding_b256_frac"] = cfg["sliding"]["frac_of_hbm_peak_median_single"]
    cfg["c3_global_b32_paged_us"] = cfg["global"]["us_per_call_median_of_50_single"]
    cfg["c3_global_b32_paged_frac"] = cfg["global"]["frac_of_hbm_peak_median_single"]
    achieved = gl_bytes / (gl_main * 1e-6) / 1e9
    trace_us, trace_box, trace_current = read_trace("global_main")
    line["roofline"] = {
        "kernel": "gqa_group_kernel<4,512,paged,bf16> (decodeGQA, B=32 paged, group mode)",
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
        "kernel_us": round(gl_main, 2), "box": box_name(),
        # the same kernel in the committed rocprofv3 trace (timed launches only)
        "trace_kernel_us": trace_us,
        "trace_frac": frac(gl_bytes, trace_us) if trace_us else None,
        "trace_box": trace_box, "trace_source_current": trace_current,
    }
    log("single-call medians: sliding %.1f us, global %.1f us" % (
        cfg["c2_sliding_b256_us"], cfg["c3_global_b32_paged_us"]))


def section_small(ctx, line):
    """The two small workloads (sliding f32 B=4, global bf16 B=4): read sets
    of about 100 MB, so each call is timed alone after a cache-evicting read."""
    torch, gqa, synth = ctx.torch, ctx.gqa, ctx.synth
    n = ctx.args.single_calls
    for name, key in zip(SMALL, ("c0", "c1")):
        log(f"{name}: {n} flushed single calls")
        c = synth.make_workload(name, seed=ctx.args.seed, device=ctx.dev, fill=0.0)
        o = torch.empty_like(c.q)
        call = ctx.decode_call(c, o, ctx.workspace(c.variant, c.B, c.cap))
        for _ in range(SECTION_WARMUP):
            call()
        warm = ctx.timer.warm(call, 20)
        cold = ctx.timer.single(call, n)
        queued = ctx.timer.queued(call, n)
        graph = ctx.timer.graph(call, 20)
        # kernel durations from the library's events, in a separate flushed pass
        # (the events add gaps between the launches of a call)
        gqa.profile_begin(2 * min(n, 20) + 4)
        ctx.timer.single(call, min(n, 20))
        main_us, comb_us = kernel_us(gqa.profile_read(), c.variant)
        nb = c.kv_bytes()
        line["config"][name] = {
            "variant": c.variant, "dtype": c.dtype, "B": c.B, "S_max": c.cap,
            "cache": "contiguous", "kv_bytes_per_call": nb,
            "plan": gqa.gqa_decode_plan(c.variant, c.B, c.cap),
            "us_per_call_after_flush_median": round(cold, 2),
            "kv_GBps_after_flush": gbps(nb, cold), "frac_of_hbm_peak_after_flush": frac(nb, cold),
            "main_kernel_us_after_flush": round(main_us, 2),
            "combine_kernel_us_after_flush": round(comb_us, 2),
            "us_per_call_after_flush_queued_median": round(queued, 2),
            "us_per_call_warm": round(warm, 2), "frac_of_hbm_peak_warm": frac(nb, warm),
            "us_per_call_graph": round(graph, 2), "frac_of_hbm_peak_graph": frac(nb, graph)}
        line["config"][f"{key}_{name}_us"] = round(cold, 2)
        line["config"][f"{key}_{name}_frac"] = frac(nb, cold)
        line["config"][f"{key}_{name}_us_graph"] = round(graph, 2)
        line["config"][f"{key}_{name}_us_after_flush_queued"] = round(queued, 2)
        del c, o


def section_window(ctx, line):
    torch, gqa = ctx.torch, ctx.gqa
    log("window sweep of the sliding geometry")
    sl = ctx.sl()
    o = torch.empty_like(sl.q)
    sweep = []
    for W in SWEEP_WINDOWS:
        call = ctx.decode_call(sl, o, ctx.workspace("sliding", sl.B, sl.cap, window=W), window=W)
        for _ in range(SECTION_WARMUP):
            call()
        us = ctx.timer.warm(call, 5)
        gqa.profile_begin(16)
        ctx.timer.warm(call, 5)
        main_us, comb_us = kernel_us(gqa.profile_read(), "sliding")
        nb = sl.kv_bytes(window=W)
        sweep.append({"window": W, "plan": gqa.gqa_decode_plan("sliding", sl.B, sl.cap, window=W),
                      "kv_bytes_per_call": nb, "us_per_call": round(us, 2),
                      "main_kernel_us": round(main_us, 2), "combine_kernel_us": round(comb_us, 2),
                      "kv_GBps": gbps(nb, us), "frac_of_hbm_peak": frac(nb, us)})
    line["config"]["sliding_window_sweep"] = sweep


def section_append(ctx, line):
    torch, gqa = ctx.torch, ctx.gqa
    log("KV append (norms + RoPE of the new token, cache write)")
    app = {}
    gen = torch.Generator(device=ctx.dev).manual_seed(ctx.args.seed + 7)
    for name, case in (("sliding_b256_contiguous", ctx.sl()), ("global_b32_paged", ctx.gl())):
        KV, D = case.KV, case.D
        tok = [torch.randn(case.B, n, D, device=ctx.dev, generator=gen).to(torch.bfloat16)
               for n in (32, KV, KV)]
        wq, wk = (torch.empty(D, device=ctx.dev).uniform_(0.2, 0.4, generator=gen)
                  .to(torch.bfloat16) for _ in range(2))
        q_out = torch.empty_like(tok[0])
        if case.variant == "sliding":
            call = lambda: gqa.gqa_append_sliding(tok[0], tok[1], tok[2], wq, wk, case.seq_lens,  # noqa: E731
                                                  case.k, case.v, block_table=case.block_table,
                                                  q_out=q_out, stream=ctx.stream)
        else:
            call = lambda: gqa.gqa_append_global(tok[0], tok[1], wq, wk, case.seq_lens, case.k,  # noqa: E731
                                                 case.v, block_table=case.block_table,
                                                 q_out=q_out, stream=ctx.stream)
        for _ in range(SECTION_WARMUP):
            call()
        us = ctx.timer.warm(call, 20)
        rows_in = 32 + KV * (2 if case.variant == "sliding" else 1)
        moved = case.B * (rows_in + 32 + 2 * KV) * D * 2 + 2 * D * 2
        app[name] = {"B": case.B, "us_per_call": round(us, 2), "bytes_per_call": moved,
                     "GBps": gbps(moved, us)}
    line["config"]["append"] = app


def section_kfv(ctx, line):
    torch, gqa = ctx.torch, ctx.gqa
    log("decodeGQA over the values-only cache (keys rebuilt from values), global B=32 paged")
    gl = ctx.gl()
    o = torch.empty_like(gl.q)
    ws = ctx.workspace("global", gl.B, gl.cap)

    def call():
        gqa.gqa_decode_global_k_eq_v_paged(gl.q, gl.v, gl.w_k, gl.block_table, gl.seq_lens,
                                           o=o, workspace=ws, stream=ctx.stream)

    for _ in range(SECTION_WARMUP):
        call()
    reps = max(3, min(ctx.args.steps, 10))
    us = ctx.timer.warm(call, reps)
    gqa.profile_begin(2 * reps + 4)
    ctx.timer.warm(call, reps)
    kprof = gqa.profile_read()
    k_main, k_comb = kprof[("global_k_eq_v", "main")], kprof[("global_k_eq_v", "combine")]
    main_us = k_main[1] / max(k_main[0], 1) * 1e3
    v_only = gl.kv_bytes() // 2  # the value rows only
    stored = line["config"].get("global", {}).get("us_per_call")
    line["config"]["global_k_eq_v"] = {
        "cache": "paged16, values only", "v_bytes_per_call": v_only,
        "us_per_call": round(us, 2), "main_kernel_us": round(main_us, 2),
        "combine_kernel_us": round(k_comb[1] / max(k_comb[0], 1) * 1e3, 2),
        "v_GBps": gbps(v_only, us), "frac_of_hbm_peak": frac(v_only, us),
        "main_kernel_frac_of_hbm_peak": frac(v_only, main_us),
        "speedup_vs_stored_keys": round(stored / us, 3) if stored else None,
        "main_kernel_hbm_traffic": read_traffic("kfv_main"),
    }


def section_ring(ctx, line):
    torch, gqa, synth = ctx.torch, ctx.gqa, ctx.synth
    log("slidingDecodeGQA over caches capped at the window (ring of 1024 slots), "
        "B=256, seq_lens U[1,262144]")
    ring_lens = synth.draw_seq_lens(("uniform", 1, 262144), 256, ctx.args.seed)
    rg = synth.make_ring_case("bf16", 256, 1024, ring_lens, seed=ctx.args.seed, device=ctx.dev,
                              fill=0.0, window=1024)
    o = torch.empty_like(rg.q)
    need = gqa.gqa_decode_sliding_ring_workspace_bytes(256, 1024, 1024)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=ctx.dev)

    def call():
        gqa.gqa_decode_sliding_ring(rg.q, rg.k, rg.v, rg.seq_lens, window=1024, o=o,
                                    workspace=ws, stream=ctx.stream)

    for _ in range(SECTION_WARMUP):
        call()
    us = ctx.timer.warm(call, max(3, min(ctx.args.steps, 10)))
    nb = int(torch.clamp(ring_lens.to(torch.int64), max=1024).sum()) * 16 * 256 * 2 * 2
    line["config"]["sliding_ring"] = {
        "B": 256, "ring_slots": 1024, "window": 1024, "seq_lens": "U[1,262144]",
        "cache_bytes": 2 * rg.k.numel() * 2, "kv_bytes_per_call": nb,
        "us_per_call": round(us, 2), "kv_GBps": gbps(nb, us), "frac_of_hbm_peak": frac(nb, us)}


def section_long(ctx, line):
    torch, gqa, synth = ctx.torch, ctx.gqa, ctx.synth
    log("one sequence of 262144 positions (paged), both geometries; warm and flushed single calls")
    b1 = {}
    n = ctx.args.single_calls
    for name in LONG:
        c = synth.make_workload(name, seed=ctx.args.seed, device=ctx.dev, fill=0.0)
        o = torch.empty_like(c.q)
        call = ctx.decode_call(c, o, ctx.workspace(c.variant, c.B, c.cap))
        for _ in range(SECTION_WARMUP):
            call()
        warm = ctx.timer.warm(call, 20)
        cold = ctx.timer.single(call, n)
        queued = ctx.timer.queued(call, n)
        graph = ctx.timer.graph(call, 20)
        gqa.profile_begin(48)
        ctx.timer.warm(call, 20)
        main_w, comb_w = kernel_us(gqa.profile_read(), c.variant)
        nb = c.kv_bytes()
        b1[name] = {"kv_bytes_per_call": nb, "plan": gqa.gqa_decode_plan(c.variant, c.B, c.cap),
                    "us_per_call": round(warm, 2), "kv_GBps": gbps(nb, warm),
                    "frac_of_hbm_peak": frac(nb, warm), "main_kernel_us": round(main_w, 2),
                    "combine_kernel_us": round(comb_w, 2),
                    "us_per_call_after_flush_median": round(cold, 2),
                    "frac_of_hbm_peak_after_flush": frac(nb, cold),
                    "us_per_call_after_flush_queued_median": round(queued, 2),
                    "us_per_call_graph": round(graph, 2), "frac_of_hbm_peak_graph": frac(nb, graph)}
        key = "c4_global" if c.variant == "global" else "c4_sliding"
        line["config"][f"{key}_b1_s262144_us"] = round(warm, 2)
        line["config"][f"{key}_b1_s262144_us_after_flush"] = round(cold, 2)
        line["config"][f"{key}_b1_s262144_us_graph"] = round(graph, 2)
        line["config"][f"{key}_b1_s262144_us_after_flush_queued"] = round(queued, 2)
        line["config"][f"{key}_b1_s262144_frac"] = frac(nb, warm)
        del c, o
    line["config"]["single_sequence_262144"] = b1


def bench_prefill(seed, dev, stream) -> dict:
    """Times each prefill workload: the call with stream events, the kernel with
    the library's own HIP events on the launch stream; the algorithmic flops
    count the unmasked (query, key) pairs."""
    import torch
    import decode_attention_slidingdecodegqa_amd as gqa
    import synth

    log("prefill / chunked prefill (MFMA-bound; algorithmic flops of the unmasked pairs)")
    pre = {}
    # the two workloads, then the sliding one at the Retrofit page's wider
    # per-layer windows (runtime-window entry point)
    runs = [(name, None) for name in sorted(synth.PREFILL_WORKLOADS)]
    runs += [("sliding_bf16_prefill_b8_past4096_chunk2048", w) for w in (2048, 4096)]
    for name, window in runs:
        pc = synth.make_prefill_workload(name, seed=seed, device=dev, fill=0.0, window=window)
        o_pf = torch.empty_like(pc.q)
        if window is not None:
            name = f"{name}_window{window}"

            def pf_call():
                gqa.gqa_prefill_sliding_window(pc.q, pc.k, pc.v, pc.cu_q, pc.seq_lens, window,
                                               block_table=pc.block_table, o=o_pf, stream=stream)
        else:
            fn = gqa.gqa_prefill_sliding if pc.variant == "sliding" else gqa.gqa_prefill_global

            def pf_call():
                fn(pc.q, pc.k, pc.v, pc.cu_q, pc.seq_lens, block_table=pc.block_table, o=o_pf,
                   stream=stream)

        for _ in range(SECTION_WARMUP):
            pf_call()
        reps = 10
        gqa.profile_begin(reps + 2)
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        for _ in range(reps):
            pf_call()
        b_ev.record(stream)
        torch.cuda.synchronize()
        pprof = gqa.profile_read()[(pc.variant, "prefill")]
        ms = a_ev.elapsed_time(b_ev) / reps
        fl = pc.flops()
        pre[name] = {"B": pc.B, "query_rows": pc.N, "seq_len": int(pc.seq_lens[0]),
                     "cache": "paged16" if pc.block_table is not None else "contiguous",
                     "us_per_call": round(ms * 1e3, 1),
                     "kernel_us": round(pprof[1] / max(pprof[0], 1) * 1e3, 1),
                     "flops_per_call": fl, "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac_of_bf16_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del pc, o_pf
    return pre


# ------------------------------------------------------------ the CPU oracle

def oracle_threads() -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return max(1, min(avail, CPU_SHARE))


def _window_rows(c, bs, window):
    """Host copy of the rows contiguous sequences bs attend to under `window`,
    re-based to position 0 (the oracle then attends to exactly these rows, in
    order)."""
    import torch
    import synth
    spans = [c.attended(b, window=window) for b in bs]
    n_max = max(1, max(L - lo for lo, L in spans))
    k = torch.zeros((len(bs), n_max, c.KV, c.D), dtype=c.k.dtype)
    v = torch.zeros_like(k)
    for i, (b, (lo, L)) in enumerate(zip(bs, spans)):
        if L > lo:
            k[i, :L - lo] = c.k[b, lo:L].cpu()
            v[i, :L - lo] = c.v[b, lo:L].cpu()
    lens = torch.tensor([L - lo for lo, L in spans], dtype=torch.int32)
    return synth.Case(c.variant, c.dtype, c.q[list(bs)].cpu(), k, v, lens, None, n_max, window)


def _paged_sequence(c, b):
    """Host copy of one paged sequence: its pages in block-table order."""
    import torch
    import synth
    L = int(c.seq_lens[b])
    lo, _ = c.attended(b)
    p0, p1 = lo // 16, (L + 15) // 16
    phys = c.block_table[b, p0:p1].to(torch.int64)
    bt = torch.full((1, c.block_table.shape[1]), -1, dtype=torch.int32)
    bt[0, p0:p1] = torch.arange(p1 - p0, dtype=torch.int32)
    return synth.Case(c.variant, c.dtype, c.q[b:b + 1].cpu(), c.k[phys].cpu(), c.v[phys].cpu(),
                      c.seq_lens[b:b + 1].cpu(), bt, c.cap, c.window)


def time_oracle(cases_iter, threads):
    """Oracle seconds over host cases built one batch at a time (building and
    copying are not timed); returns (K/V bytes, seconds)."""
    import oracle
    import synth
    nbytes, secs = 0, 0.0
    for c in cases_iter:
        bt = None if c.block_table is None else synth.to_numpy(c.block_table)
        args = (synth.to_numpy(c.q), synth.to_numpy(c.k), synth.to_numpy(c.v),
                synth.to_numpy(c.seq_lens))
        t0 = time.perf_counter()
        oracle.gqa_decode(c.variant, *args, block_table=bt, nthreads=threads)
        secs += time.perf_counter() - t0
        nbytes += c.kv_bytes()
    return nbytes, secs


def cpu_baseline(ctx, line):
    """The fp64 oracle, as it stands, on the host cores: the whole step's
    workload (every sequence of both calls), then configs 0 and 1 on one
    thread and on all threads."""
    threads = oracle_threads()
    sl, gl = ctx.sl(), ctx.gl()
    log(f"timing the fp64 oracle on the step workload ({threads} threads)")
    sl_iter = (_window_rows(sl, list(range(b0, min(sl.B, b0 + 16))), 1024)
               for b0 in range(0, sl.B, 16))
    gl_iter = (_paged_sequence(gl, b) for b in range(gl.B))
    nb1, s1 = time_oracle(sl_iter, threads)
    nb2, s2 = time_oracle(gl_iter, threads)
    nb, secs = nb1 + nb2, s1 + s2
    small = {}
    for name in SMALL:
        c = ctx.synth.make_workload(name, seed=ctx.args.seed, device="cpu", fill=0.0)
        for t in (1, threads):
            b, s = time_oracle([c], t)
            small[f"{name}_{t}thread{'s' if t > 1 else ''}"] = {
                "kv_bytes": b, "us_per_call": round(s * 1e6, 1), "GBps": round(b / s / 1e9, 3)}
    line["cpu_baseline"] = {
        "value": round(nb / secs / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"fp64 C oracle on the whole step workload (all 32 heads of all 256 sliding "
                   f"and 32 global sequences): {nb / 1e9:.2f} GB of K/V in {secs:.2f} s of "
                   f"oracle time on {threads} threads; host copies not timed"),
        "threads": threads, "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "us_per_step": round(secs * 1e6, 1),
        "small_workloads": small,
    }


# ----------------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.skip, args.take), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this decode-attention library runs on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import decode_attention_slidingdecodegqa_amd as gqa
    gqa.library()
    if args.copy_probe:
        print(json.dumps(hbm_probes(args.copy_probe)), flush=True)
        return
    dev = torch.device("cuda:0")
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(args.seed, dev, torch.cuda.current_stream(dev))}),
              flush=True)
        return
    only = [s for s in args.only.split(",") if s]
    unknown = set(only) - set(SECTIONS)
    if unknown:
        print(f"bench.py: unknown sections {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)

    ctx = Ctx(args)
    line = {
        "metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; unit-RMS values, RMS-normed weighted q/k)",
        "config": {"workload": f"{SLIDING} + {GLOBAL}", "box": box_name(),
                   "sections": ",".join(only)},
    }
    runners = {"step": section_step, "small": section_small, "window": section_window,
               "append": section_append, "kfv": section_kfv, "ring": section_ring,
               "long": section_long}
    for name in SECTIONS:
        if name not in only:
            continue
        if name in runners:
            runners[name](ctx, line)
        elif name == "prefill":
            line["config"]["prefill"] = bench_prefill(args.seed, dev, ctx.stream)
        elif name == "probe":
            log("measuring the plain read stream (4 GiB)")
            ctx.timer.release()
            probes = hbm_probes(4 << 30)
            if "roofline" in line:
                line["roofline"]["measured_read_stream_GBps"] = probes["read_GBps"]
                line["roofline"]["frac_of_measured_read_stream"] = round(
                    line["roofline"]["achieved"] / probes["read_GBps"], 4)
            line["config"]["measured_read_stream_GBps"] = probes["read_GBps"]
    ctx.timer.release()
    if not args.no_cpu_baseline and "step" in only:
        cpu_baseline(ctx, line)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
