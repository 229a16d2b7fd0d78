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
dominant kernel against the 8 TB/s HBM3E peak, and the fp64 CPU oracle timed on
a bounded sample of the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
# runtime windows of the sliding geometry measured beside the step (per-layer
# windows of the Retrofit Plan page's progressive window table)
SWEEP_WINDOWS = (2048, 4096, 8192)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_sliding_b256_global_b32_paged.txt")
# the sources of the decode and append kernels (the profiled ones)
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_slidingdecodegqa_amd", "csrc", f)
                  for f in ("gqa_common.h", "gqa_decode.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (e.g. under a profiler)")
    ap.add_argument("--cpu-sample-seqs", type=str, default="64,8",
                    help="sequences of the sliding,global workloads the oracle is timed on")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run the library's plain read stream and plain copy over BYTES "
                         "bytes (calibrates a profiler's HBM byte counters) and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the prefill workloads (one JSON line) and exit")
    return ap.parse_args()


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


def source_hash() -> str:
    """sha256 over the decode kernels' sources, in order."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(key: str = "global_main"):
    """HBM bytes per launch of a kernel (global_main: the dominant kernel) from
    committed rocprofv3 --pmc runs, valid only if taken on the current kernel
    source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = v
    if vals.get("source_sha256") != source_hash():
        return None
    try:
        return float(vals[f"{key}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def oracle_sample(sl_case, gl_case, n_sl, n_gl, threads):
    """Time the fp64 oracle on whole sequences of both workloads (all 32 heads)."""
    import torch
    import oracle
    import synth

    def sub_contig(c, bs):
        out = []
        for b in bs:
            out.append(synth.Case(c.variant, c.dtype, c.q[b:b + 1].cpu(), c.k[b:b + 1].cpu(),
                                  c.v[b:b + 1].cpu(), c.seq_lens[b:b + 1].cpu(), None, c.cap,
                                  c.window))
        return out

    def sub_paged(c, bs):
        out = []
        bt = c.block_table.cpu()
        for b in bs:
            L = int(c.seq_lens[b])
            npg = (L + 15) // 16
            phys = bt[b, :npg].to(c.k.device, torch.int64)
            kb, vb = c.k[phys].cpu(), c.v[phys].cpu()
            tb = torch.full((1, bt.shape[1]), -1, dtype=torch.int32)
            tb[0, :npg] = torch.arange(npg, dtype=torch.int32)
            out.append(synth.Case(c.variant, c.dtype, c.q[b:b + 1].cpu(), kb, vb,
                                  c.seq_lens[b:b + 1].cpu(), tb, c.cap, c.window))
        return out

    cases = sub_contig(sl_case, range(n_sl)) + sub_paged(gl_case, range(n_gl))
    nbytes = sum(c.kv_bytes() for c in cases)
    t0 = time.perf_counter()
    for c in cases:
        bt = None if c.block_table is None else synth.to_numpy(c.block_table)
        oracle.gqa_decode(c.variant, synth.to_numpy(c.q), synth.to_numpy(c.k),
                          synth.to_numpy(c.v), synth.to_numpy(c.seq_lens), block_table=bt,
                          nthreads=threads)
    dt = time.perf_counter() - t0
    return nbytes, dt


# untimed calls before each timed section after the step: the first calls
# after a switch of workload run measurably slower
SECTION_WARMUP = 10


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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this decode-attention library runs on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        print(json.dumps(hbm_probes(args.copy_probe)), flush=True)
        return
    if args.prefill_only:
        import torch
        import decode_attention_slidingdecodegqa_amd as gqa
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        gqa.library()
        dev = torch.device("cuda:0")
        print(json.dumps({"prefill": bench_prefill(args.seed, dev, torch.cuda.current_stream(dev))}),
              flush=True)
        return

    import torch
    import decode_attention_slidingdecodegqa_amd as gqa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gqa.library()
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    log("generating the sliding B=256 contiguous cache (rows drawn for the widest window)")
    sl = synth.make_workload(SLIDING, seed=args.seed, device=dev, fill=0.0,
                             window=max(SWEEP_WINDOWS))
    log("generating the global B=32 paged cache")
    gl = synth.make_workload(GLOBAL, seed=args.seed, device=dev, fill=0.0)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f} s")
    sl_bytes, gl_bytes = sl.kv_bytes(window=1024), gl.kv_bytes()

    o_sl = torch.empty_like(sl.q)
    o_gl = torch.empty_like(gl.q)
    ws_sl_n = gqa.gqa_decode_workspace_bytes("sliding", sl.B, sl.cap)
    ws_gl_n = gqa.gqa_decode_workspace_bytes("global", gl.B, gl.cap)
    ws_sl = torch.empty(max(ws_sl_n, 256), dtype=torch.uint8, device=dev)
    ws_gl = torch.empty(max(ws_gl_n, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gqa.gqa_decode_sliding(sl.q, sl.k, sl.v, sl.seq_lens, o=o_sl, workspace=ws_sl,
                               stream=stream)
        gqa.gqa_decode_global_paged(gl.q, gl.k, gl.v, gl.block_table, gl.seq_lens, o=o_gl,
                                    workspace=ws_gl, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warm-up done ({args.warmup} steps)")

    gqa.profile_begin(4 * args.steps + 8)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    prof = gqa.profile_read()
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step")

    def avg(key):
        n, t = prof[key]
        return t / n if n else 0.0

    sl_main_ms = avg(("sliding", "main"))
    sl_comb_ms = avg(("sliding", "combine"))
    sl_ms = sl_main_ms + sl_comb_ms
    gl_split_ms = avg(("global", "main"))
    gl_comb_ms = avg(("global", "combine"))
    gl_ms = gl_split_ms + gl_comb_ms
    total_bytes = sl_bytes + gl_bytes
    value = total_bytes / (ms_step * 1e-3) / 1e9
    achieved = gl_bytes / (gl_split_ms * 1e-3) / 1e9
    traffic = read_traffic()

    plan_gl = gqa.gqa_decode_plan("global", gl.B, gl.cap)
    plan_sl = gqa.gqa_decode_plan("sliding", sl.B, sl.cap)
    config = {
        "workload": f"{SLIDING} + {GLOBAL}",
        "sliding": {
            "B": sl.B, "S_max": sl.cap, "kv_heads": 16, "head_dim": 256, "window": 1024,
            "cache": "contiguous", "kv_bytes_per_call": sl_bytes,
            "us_per_call": round(sl_ms * 1e3, 2),
            "main_kernel_us": round(sl_main_ms * 1e3, 2),
            "combine_kernel_us": round(sl_comb_ms * 1e3, 2),
            "kv_GBps": round(sl_bytes / (sl_ms * 1e-3) / 1e9, 1) if sl_ms else None,
            "frac_of_hbm_peak": round(sl_bytes / (sl_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            if sl_ms else None,
            "plan": plan_sl,
        },
        "global": {
            "B": gl.B, "max_pages": gl.block_table.shape[1], "num_pages": gl.k.shape[0],
            "kv_heads": 4, "head_dim": 512, "cache": "paged16", "kv_bytes_per_call": gl_bytes,
            "us_per_call": round(gl_ms * 1e3, 2),
            "main_kernel_us": round(gl_split_ms * 1e3, 2),
            "combine_kernel_us": round(gl_comb_ms * 1e3, 2),
            "kv_GBps": round(gl_bytes / (gl_ms * 1e-3) / 1e9, 1) if gl_ms else None,
            "frac_of_hbm_peak": round(gl_bytes / (gl_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            if gl_ms else None,
            "plan": plan_gl,
        },
    }
    # each call also timed on its own (events around one call, the stream
    # drained in between): the median of 50, after the timed steps above
    def median_single(call, n=50):
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = []
        for _ in range(n):
            a_ev.record(stream)
            call()
            b_ev.record(stream)
            torch.cuda.synchronize()
            t.append(a_ev.elapsed_time(b_ev))
        t.sort()
        return t[len(t) // 2]

    for name, call, nb in (
            ("sliding", lambda: gqa.gqa_decode_sliding(sl.q, sl.k, sl.v, sl.seq_lens, o=o_sl,
                                                       workspace=ws_sl, stream=stream), sl_bytes),
            ("global", lambda: gqa.gqa_decode_global_paged(gl.q, gl.k, gl.v, gl.block_table,
                                                           gl.seq_lens, o=o_gl, workspace=ws_gl,
                                                           stream=stream), gl_bytes)):
        med = median_single(call)
        config[name]["us_per_call_median_of_50_single"] = round(med * 1e3, 2)
        config[name]["frac_of_hbm_peak_median_single"] = round(
            nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    log("single-call medians: sliding %.1f us, global %.1f us" % (
        config["sliding"]["us_per_call_median_of_50_single"],
        config["global"]["us_per_call_median_of_50_single"]))

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; unit-RMS values, RMS-normed weighted q/k)",
        "config": config,
        "roofline": {
            "kernel": "gqa_stream_kernel<4,512,paged,bf16> (decodeGQA, B=32 paged)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    log("window sweep of the sliding geometry")
    sweep = []
    for W in SWEEP_WINDOWS:
        need = gqa.gqa_decode_workspace_bytes("sliding", sl.B, sl.cap, window=W)
        ws_w = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        for _ in range(SECTION_WARMUP):
            gqa.gqa_decode_sliding_window(sl.q, sl.k, sl.v, sl.seq_lens, W, o=o_sl,
                                          workspace=ws_w, stream=stream)
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a_ev.record(stream)
        for _ in range(reps):
            gqa.gqa_decode_sliding_window(sl.q, sl.k, sl.v, sl.seq_lens, W, o=o_sl,
                                          workspace=ws_w, stream=stream)
        b_ev.record(stream)
        torch.cuda.synchronize()
        ms = a_ev.elapsed_time(b_ev) / reps
        nb = sl.kv_bytes(window=W)
        sweep.append({"window": W, "plan": gqa.gqa_decode_plan("sliding", sl.B, sl.cap, window=W),
                      "kv_bytes_per_call": nb, "us_per_call": round(ms * 1e3, 2),
                      "kv_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                      "frac_of_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        del ws_w
    line["config"]["sliding_window_sweep"] = sweep
    log("KV append (norms + RoPE of the new token, cache write)")
    app = {}
    gen = torch.Generator(device=dev).manual_seed(args.seed + 7)
    for name, case in (("sliding_b256_contiguous", sl), ("global_b32_paged", gl)):
        KV, D = case.KV, case.D
        tok = [torch.randn(case.B, n, D, device=dev, generator=gen).to(torch.bfloat16)
               for n in (32, KV, KV)]
        wq, wk = (torch.empty(D, device=dev).uniform_(0.2, 0.4, generator=gen)
                  .to(torch.bfloat16) for _ in range(2))
        q_out = torch.empty_like(tok[0])
        if case.variant == "sliding":
            call = lambda: gqa.gqa_append_sliding(tok[0], tok[1], tok[2], wq, wk, case.seq_lens,
                                                  case.k, case.v, block_table=case.block_table,
                                                  q_out=q_out, stream=stream)
        else:
            call = lambda: gqa.gqa_append_global(tok[0], tok[1], wq, wk, case.seq_lens, case.k,
                                                 case.v, block_table=case.block_table,
                                                 q_out=q_out, stream=stream)
        for _ in range(SECTION_WARMUP):
            call()
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        a_ev.record(stream)
        for _ in range(reps):
            call()
        b_ev.record(stream)
        torch.cuda.synchronize()
        ms = a_ev.elapsed_time(b_ev) / reps
        rows_in = 32 + KV * (2 if case.variant == "sliding" else 1)
        moved = case.B * (rows_in + 32 + 2 * KV) * D * 2 + 2 * D * 2
        app[name] = {"B": case.B, "us_per_call": round(ms * 1e3, 2), "bytes_per_call": moved,
                     "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
    line["config"]["append"] = app
    log("decodeGQA over the values-only cache (keys rebuilt from values), global B=32 paged")
    o_kv = torch.empty_like(gl.q)

    def kfv_call():
        gqa.gqa_decode_global_k_eq_v_paged(gl.q, gl.v, gl.w_k, gl.block_table, gl.seq_lens,
                                           o=o_kv, workspace=ws_gl, stream=stream)

    for _ in range(SECTION_WARMUP):
        kfv_call()
    reps = max(3, min(args.steps, 10))
    gqa.profile_begin(2 * reps + 4)
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record(stream)
    for _ in range(reps):
        kfv_call()
    b_ev.record(stream)
    torch.cuda.synchronize()
    kprof = gqa.profile_read()
    ms = a_ev.elapsed_time(b_ev) / reps
    k_main = kprof[("global_k_eq_v", "main")]
    k_comb = kprof[("global_k_eq_v", "combine")]
    kv_only = gl_bytes // 2  # the value rows only
    line["config"]["global_k_eq_v"] = {
        "cache": "paged16, values only", "v_bytes_per_call": kv_only,
        "us_per_call": round(ms * 1e3, 2),
        "main_kernel_us": round(k_main[1] / max(k_main[0], 1) * 1e3, 2),
        "combine_kernel_us": round(k_comb[1] / max(k_comb[0], 1) * 1e3, 2),
        "v_GBps": round(kv_only / (ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(kv_only / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "speedup_vs_stored_keys": round(gl_ms / ms, 3) if ms else None,
        "main_kernel_hbm_traffic": read_traffic("kfv_main"),
    }
    log("slidingDecodeGQA over caches capped at the window (ring of 1024 slots), "
        "B=256, seq_lens U[1,262144]")
    ring_lens = synth.draw_seq_lens(("uniform", 1, 262144), 256, args.seed)
    rg = synth.make_ring_case("bf16", 256, 1024, ring_lens, seed=args.seed, device=dev,
                              fill=0.0, window=1024)
    o_rg = torch.empty_like(rg.q)
    ws_rg_n = gqa.gqa_decode_sliding_ring_workspace_bytes(256, 1024, 1024)
    ws_rg = torch.empty(max(ws_rg_n, 256), dtype=torch.uint8, device=dev)

    def ring_call():
        gqa.gqa_decode_sliding_ring(rg.q, rg.k, rg.v, rg.seq_lens, window=1024, o=o_rg,
                                    workspace=ws_rg, stream=stream)

    for _ in range(SECTION_WARMUP):
        ring_call()
    reps = max(3, min(args.steps, 10))
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record(stream)
    for _ in range(reps):
        ring_call()
    b_ev.record(stream)
    torch.cuda.synchronize()
    ms = a_ev.elapsed_time(b_ev) / reps
    rg_bytes = int(torch.clamp(ring_lens.to(torch.int64), max=1024).sum()) * 16 * 256 * 2 * 2
    line["config"]["sliding_ring"] = {
        "B": 256, "ring_slots": 1024, "window": 1024, "seq_lens": "U[1,262144]",
        "cache_bytes": 2 * rg.k.numel() * 2, "kv_bytes_per_call": rg_bytes,
        "us_per_call": round(ms * 1e3, 2), "kv_GBps": round(rg_bytes / (ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(rg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del rg, o_rg, ws_rg
    log("one sequence of 262144 positions (paged), both geometries; also cold single calls")
    b1 = {}
    for name in ("global_bf16_b1_paged_s262144", "sliding_bf16_b1_paged_s262144"):
        c1 = synth.make_workload(name, seed=args.seed, device=dev, fill=0.0)
        fn1 = gqa.gqa_decode_global_paged if c1.variant == "global" else gqa.gqa_decode_sliding_paged
        o1 = torch.empty_like(c1.q)
        ws1 = torch.empty(max(gqa.gqa_decode_workspace_bytes(c1.variant, c1.B, c1.cap), 256),
                          dtype=torch.uint8, device=dev)

        def b1_call():
            fn1(c1.q, c1.k, c1.v, c1.block_table, c1.seq_lens, o=o1, workspace=ws1, stream=stream)

        for _ in range(SECTION_WARMUP):
            b1_call()
        reps = 20
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        for _ in range(reps):
            b1_call()
        b_ev.record(stream)
        torch.cuda.synchronize()
        ms = a_ev.elapsed_time(b_ev) / reps
        # single calls, each after a 2 GiB read that evicts the caches (the
        # sliding window is 16 MiB): the median of 50, outside any warm chain.
        # A read leaves no dirty lines for the call to write back.
        flush = torch.ones(512 << 20, dtype=torch.float32, device=dev)
        single = []
        for _ in range(50):
            flush.sum()
            torch.cuda.synchronize()
            a_ev.record(stream)
            b1_call()
            b_ev.record(stream)
            torch.cuda.synchronize()
            single.append(a_ev.elapsed_time(b_ev))
        del flush
        single.sort()
        ms_cold = single[len(single) // 2]
        by = c1.kv_bytes()
        b1[name] = {"kv_bytes_per_call": by, "us_per_call": round(ms * 1e3, 2),
                    "kv_GBps": round(by / (ms * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "us_per_call_after_flush_median": round(ms_cold * 1e3, 2),
                    "frac_of_hbm_peak_after_flush": round(by / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del c1, o1, ws1
    line["config"]["single_sequence_262144"] = b1
    line["config"]["prefill"] = bench_prefill(args.seed, dev, stream)
    log("measuring the plain read stream (4 GiB)")
    probes = hbm_probes(4 << 30)
    line["roofline"]["measured_read_stream_GBps"] = probes["read_GBps"]
    line["roofline"]["frac_of_measured_read_stream"] = round(achieved / probes["read_GBps"], 4)
    if not args.no_cpu_baseline:
        n_sl, n_gl = (int(x) for x in args.cpu_sample_seqs.split(","))
        threads = min(os.cpu_count() or 1, 16)
        log(f"timing the fp64 oracle on {n_sl} sliding + {n_gl} global sequences, "
            f"{threads} threads")
        nb, dt = oracle_sample(sl, gl, n_sl, n_gl, threads)
        line["cpu_baseline"] = {
            "value": round(nb / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 C oracle, all 32 heads of the first {n_sl} sequences of the "
                       f"sliding B=256 cache and the first {n_gl} of the global B=32 paged "
                       f"cache: {nb / 1e9:.3f} GB of K/V in {dt:.2f} s"),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
