#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

Headline: split-KV GQA decode (partial kernel + LSE merge) on the
Llama-3-8B-shaped workload -- 16 requests, 32 query / 8 KV heads, head_dim
128, 4096 keys each, bf16 in / fp32 accumulate -- reported as whole-step
HBM throughput in GB/s of algorithmic bytes (K + V + Q read, O + LSE
written, indptr read), with inputs resident in HBM before timing starts.
Three copies of K/V are rotated across steps so that consecutive steps do
not hit the 256 MB Infinity Cache (one copy of K + V is 268 MB).

Also measured in the same run (reported under "also"): causal prefill
(B 2, L 4096, 32/8 heads, D 128, bf16) in TFLOP/s of the lower triangle,
ragged serving-like decode (64 requests, 64/8 heads, lengths log-uniform in
[128, 32768]; flat split plan, chunk plan for comparison) in GB/s, append
prefill, MLA decode (absorbed form, 576-element cache rows; 16 heads x 32
requests x 4096 tokens, and 128 heads with ragged lengths) in GB/s, and
block-sparse prefill (B 1, L 4096, 16 heads, D 64, fp16) in TFLOP/s at
outer-tile granularity.

Prints one JSON line on stdout (progress goes to stderr).
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
METRIC = "split-KV GQA decode HBM GB/s (% peak); causal prefill TFLOP/s (% MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--splits", type=int, default=0, help="force the decode split count")
    p.add_argument("--only", choices=["decode", "prefill", "ragged", "ragged_flat", "mla", "mla_ragged", "bsr", "bsr_heads", "append",
                                      "copy"],
                   default=None,
                   help="time one workload only (for profiler runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-also", action="store_true", help="skip the secondary workloads")
    p.add_argument("--warm-seconds", type=float, default=0.3,
                   help="untimed run time of each workload before its timed steps (GPU clock warm-up)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_partial_traffic.json"))
    return p.parse_args()


class Timer:
    """HIP events recorded on the stream the library launches on.

    Before the timed steps: the W warm-up steps, then more untimed steps of
    the same work until ``warm_s`` seconds have passed, so that the GPU has
    reached its working clock (a few milliseconds of steps do not; a fresh
    process measured the causal prefill 10% slower without this)."""

    def __init__(self, torch, stream, warm_s=0.3):
        self.torch, self.stream, self.warm_s = torch, stream, warm_s

    def run(self, fn, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0, i = time.perf_counter(), warmup
        while time.perf_counter() - t0 < self.warm_s:
            for _ in range(8):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t0 = time.perf_counter()
        for k in range(steps):
            ev[k][0].record(self.stream)
            fn(i + k)
            ev[k][1].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [a.elapsed_time(b) for a, b in ev]
        return ms, wall


def median(x):
    s = sorted(x)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def decode_bytes(B, Hq, Hkv, D, total_kv, elem):
    kv = 2 * total_kv * Hkv * D * elem
    q = B * Hq * D * elem
    o = B * Hq * D * elem
    lse = B * Hq * 4
    indptr = (B + 1) * 4
    return kv, q, o, lse, indptr


def bench_decode(torch, ra, synth, wname, args, timer, rotate=3):
    w = synth.workload(wname)
    inp = w.make("cuda:0")
    dev = torch.device("cuda:0")
    lengths = inp["lengths"]
    max_len = max(lengths)
    total = sum(lengths)
    q = inp["q"].to(dev)
    kvp = inp["kv_indptr"].to(dev)
    sets = [(inp["k"].to(dev), inp["v"].to(dev))]
    for _ in range(rotate - 1):
        sets.append((sets[0][0].clone(), sets[0][1].clone()))
    s = args.splits or ra.attn_decode_choose_splits(w.B, w.Hq, w.Hkv, w.D, total, max_len)
    ws = torch.empty(ra.attn_decode_workspace_bytes(w.B, w.Hq, w.D, s), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        k, v = sets[i % rotate]
        ra.attn_decode_splitkv(q, k, v, kvp, max_len, num_splits=s, o=o, lse=lse, workspace=ws,
                               stream=stream)

    # one step = the Split partial kernel + the merge kernel, both on `stream`
    ms, wall = timer.run(step, args.steps, args.warmup)
    # the partial kernel alone (the step's first kernel, every split kept as a
    # partial), timed the same way: the dominant kernel's launch duration
    rows = w.B * w.Hq
    op = torch.empty((s, rows, w.D), dtype=torch.float32, device=dev)
    mp = torch.empty((s, rows), dtype=torch.float32, device=dev)
    lp = torch.empty((s, rows), dtype=torch.float32, device=dev)

    def partials(i):
        k, v = sets[i % rotate]
        ra.attn_decode_partials(q, k, v, kvp, max_len, s, o_part=op, m_part=mp, l_part=lp,
                                stream=stream)

    ms_k, _ = timer.run(partials, args.steps, args.warmup)
    # the same step captured ten at a time in a HIP graph (one graph per
    # K/V copy order), as a serving loop would launch it: per-step time
    graph_ms = None
    if rotate > 1:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graphs = []
        with torch.cuda.stream(side):
            for c in range(rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    for t in range(10):
                        k, v = sets[(c + t) % rotate]
                        ra.attn_decode_splitkv(q, k, v, kvp, max_len, num_splits=s, o=o, lse=lse,
                                               workspace=ws, stream=torch.cuda.current_stream())
                graphs.append(g)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        ms_g, _ = timer.run(lambda i: graphs[i % rotate].replay(), max(args.steps // 10, 3),
                            max(args.warmup // 10, 1))
        graph_ms = median(ms_g) / 10
    elem = q.element_size()
    kvb, qb, ob, lb, ib = decode_bytes(w.B, w.Hq, w.Hkv, w.D, total, elem)
    step_ms = median(ms)
    kernel_ms = median(ms_k)
    step_bytes = kvb + qb + ob + lb + ib
    kernel_bytes = kvb + qb + ib  # what the partial kernel must read
    return dict(workload=wname, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, total_kv=total,
                max_kv_len=max_len, splits=s, chunk=-(-max_len // s), dtype=str(q.dtype),
                step_ms=step_ms, step_ms_p10=sorted(ms)[len(ms) // 10],
                step_ms_p90=sorted(ms)[(9 * len(ms)) // 10], step_bytes=step_bytes,
                kv_bytes=kvb, gbs=step_bytes / step_ms / 1e6, kernel_ms=kernel_ms,
                kernel_bytes=kernel_bytes, kernel_gbs=kernel_bytes / kernel_ms / 1e6,
                wall_s=wall, kv_copies_rotated=rotate, graph_step_ms=graph_ms)


def bench_decode_flat(torch, ra, synth, wname, args, timer):
    """Split-KV decode with the flat plan (packed key rows cut into equal
    pieces), whole step: pieces kernel + merge."""
    w = synth.workload(wname)
    inp = w.make("cuda:0")
    dev = torch.device("cuda:0")
    lengths = inp["lengths"]
    max_len, total = max(lengths), sum(lengths)
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    kvp = inp["kv_indptr"].to(dev)
    P = ra.attn_decode_flat_pieces(w.B, w.Hq, w.Hkv, w.D, k.shape[0])
    ws = torch.empty(max(ra.attn_decode_flat_workspace_bytes(w.B, w.Hq, w.D, max_len, k.shape[0], P),
                         256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ms, _ = timer.run(lambda i: ra.attn_decode_splitkv_flat(q, k, v, kvp, max_len, num_pieces=P,
                                                            o=o, lse=lse, workspace=ws,
                                                            stream=stream), args.steps, args.warmup)
    kvb, qb, ob, lb, ib = decode_bytes(w.B, w.Hq, w.Hkv, w.D, total, q.element_size())
    t = median(ms)
    return dict(workload=wname, pieces=P, piece_len=-(-k.shape[0] // P), step_ms=t,
                gbs=(kvb + qb + ob + lb + ib) / t / 1e6)


def bench_mla(torch, ra, synth, wname, args, timer):
    """MLA decode (absorbed form), whole step: chunk kernel + merge.  Bytes:
    cache rows (576 x 2 B per token, read once for keys and values), q,
    o (512 wide), lse, indptr."""
    w = synth.workload(wname)
    inp = w.make("cuda:0")
    q, kv, kvp = inp["q"], inp["kv"], inp["kv_indptr"]
    L = inp["lengths"]
    max_len, total = max(L), sum(L)
    s = ra.attn_mla_decode_choose_splits(w.B, w.Hq, total, max_len)
    ws = torch.empty(max(ra.attn_mla_decode_workspace_bytes(w.B, w.Hq, s), 256), dtype=torch.uint8,
                     device=q.device)
    o = torch.empty((w.B, w.Hq, 512), dtype=q.dtype, device=q.device)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    ms, _ = timer.run(lambda i: ra.attn_mla_decode(q, kv, kvp, max_len, w.scale, num_splits=s, o=o,
                                                   lse=lse, workspace=ws, stream=stream),
                      args.steps, args.warmup)
    t = median(ms)
    byt = total * 576 * 2 + w.B * w.Hq * (576 * 2 + 512 * 2 + 4) + 4 * (w.B + 1)
    flops = 2 * w.Hq * total * (576 + 512)
    # the library runs its 64-head kernel when H is a multiple of 64
    kernel = "mla_wide_kernel" if w.Hq >= 64 and w.Hq % 64 == 0 else "mla_decode_kernel"
    return dict(workload=wname, B=w.B, H=w.Hq, total_kv=total, max_kv_len=max_len, splits=s,
                kernel=kernel, ms=t, bytes=byt, gbs=byt / t / 1e6,
                frac=byt / t / 1e6 / HBM_PEAK_GBS, tflops=flops / t / 1e9,
                frac_mfma=flops / t / 1e9 / MFMA_BF16_PEAK_TFS)


def causal_flops(B, Hq, L, D):
    # QK^T and PV over the lower triangle including the diagonal: 2 * 2 * D per pair
    return 4 * D * (L * (L + 1) // 2) * B * Hq


def bench_prefill(torch, ra, synth, args, timer):
    w = synth.workload("causal_prefill_bf16")
    inp = w.make("cuda:0")
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qo, kv = inp["qo_indptr"].to(dev), inp["kv_indptr"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], w.Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ms, wall = timer.run(lambda i: ra.attn_prefill(q, k, v, qo, kv, w.L, w.L, causal=True, o=o,
                                                   lse=lse, stream=stream), args.steps, args.warmup)
    flops = causal_flops(w.B, w.Hq, w.L, w.D)
    t = median(ms)
    return dict(workload=w.name, B=w.B, L=w.L, Hq=w.Hq, Hkv=w.Hkv, D=w.D, dtype="bf16",
                ms=t, flops=flops, tflops=flops / t / 1e9,
                frac=flops / t / 1e9 / MFMA_BF16_PEAK_TFS)


def append_flops(B, Hq, Lq, L, D):
    # bottom-right causal: new token t of Lq sees L - Lq + t + 1 keys
    pairs = sum(L - Lq + t + 1 for t in range(Lq))
    return 4 * D * pairs * B * Hq


def bench_append(torch, ra, synth, args, timer):
    """Append / chunked prefill: the split-KV prefill at its automatic split
    count, and the unsplit kernel on the same inputs for comparison."""
    w = synth.workload("append_prefill_bf16")
    inp = w.make("cuda:0")
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qo, kv = inp["qo_indptr"].to(dev), inp["kv_indptr"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], w.Hq), dtype=torch.float32, device=dev)
    s = ra.attn_prefill_choose_splits(w.B, w.Hq, w.Hkv, w.D, w.Lq, w.L)
    ws = torch.empty(max(ra.attn_prefill_workspace_bytes(q.shape[0], w.Hq, w.D, s), 256),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ms, _ = timer.run(lambda i: ra.attn_prefill_splitkv(q, k, v, qo, kv, w.Lq, w.L, causal=True,
                                                        num_splits=s, o=o, lse=lse, workspace=ws,
                                                        stream=stream), args.steps, args.warmup)
    ms1, _ = timer.run(lambda i: ra.attn_prefill(q, k, v, qo, kv, w.Lq, w.L, causal=True, o=o,
                                                 lse=lse, stream=stream), args.steps, args.warmup)
    flops = append_flops(w.B, w.Hq, w.Lq, w.L, w.D)
    t, t1 = median(ms), median(ms1)
    return dict(workload=w.name, B=w.B, Lq=w.Lq, L=w.L, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                dtype="bf16", splits=s, ms=t, flops=flops, tflops=flops / t / 1e9,
                frac=flops / t / 1e9 / MFMA_BF16_PEAK_TFS, ms_unsplit=t1,
                tflops_unsplit=flops / t1 / 1e9)


def bench_bsr(torch, ra, synth, args, timer, name="bsr_prefill_fp16"):
    w = synth.workload(name)
    inp = w.make("cuda:0")
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    m = ra.attn_bsr_encode_host(inp["mask"])
    enc_s = time.perf_counter() - t0
    md = m.to(dev)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.L, w.Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    plan = m.plan(w.D, w.Hq, w.B)
    plan_s = time.perf_counter() - t0
    times = {}
    for kern in ("block", "row"):
        ms, _ = timer.run(lambda i: ra.attn_prefill_bsr(q, k, v, md, o=o, lse=lse, stream=stream,
                                                        kernel=kern), args.steps, args.warmup)
        times[kern] = median(ms)
    # every mask serves Hq / num_masks heads
    hpm = w.Hq // m.num_masks
    n_ot = m.nnz_full + m.nnz_part
    flops_ot = 4 * w.D * 64 * 64 * n_ot * hpm * w.B
    flops_rows = 4 * w.D * 16 * 16 * plan["row_blocks"] * hpm * w.B
    valid = int(inp["mask"].to(torch.int64).sum())
    flops_valid = 4 * w.D * valid * hpm * w.B
    t = times[plan["kernel"]]  # what kernel="auto" runs
    return dict(workload=w.name, B=w.B, L=w.L, H=w.Hq, D=w.D, dtype="fp16", ms=t,
                kernel=plan["kernel"], ms_block=times["block"], ms_row=times["row"],
                num_masks=m.num_masks, nnz_full=m.nnz_full, nnz_part=m.nnz_part,
                row_blocks=plan["row_blocks"], model_block_us=plan["block_cost"],
                model_row_us=plan["row_cost"],
                density=valid / (w.L * w.L * m.num_masks), flops_ot=flops_ot,
                tflops_ot=flops_ot / times["block"] / 1e9,
                tflops_rows=flops_rows / times["row"] / 1e9,
                tflops_valid=flops_valid / t / 1e9,
                frac_ot=flops_ot / times["block"] / 1e9 / MFMA_BF16_PEAK_TFS,
                host_encode_s=enc_s, host_plan_s=plan_s)


def bench_copy(torch, args, timer):
    """A plain device copy of known size: the calibration of the HBM byte counters."""
    n = 1 << 30
    dev = torch.device("cuda:0")
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    ms, _ = timer.run(lambda i: b.copy_(a), args.steps, args.warmup)
    return dict(bytes_read=n, bytes_written=n, ms=median(ms), gbs=2 * n / median(ms) / 1e6)


def cpu_baseline(torch, synth, budget_s):
    """The fp64 oracle on a bounded sample of the headline decode workload."""
    import oracle
    w = synth.workload("llama3_8b_decode_bf16")
    inp = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in w.make("cuda:0").items()}
    threads = len(os.sched_getaffinity(0))
    threads = min(threads, 16)
    B, Hq = w.B, w.Hq
    qo = list(range(B + 1))
    # sample: (request, query head) rows in order, wrapping around, in
    # batches grown until one batch takes about a second, for about budget_s
    rows_all = [(b, h) for b in range(B) for h in range(Hq)]
    n, pos, done = 8, 0, 0
    t0 = time.perf_counter()
    while True:
        sel = [rows_all[(pos + k) % len(rows_all)] for k in range(n)]
        pos += n
        tb = time.perf_counter()
        oracle.attention(inp["q"], inp["k"], inp["v"], qo, inp["kv_indptr"], w.scale,
                         rows=torch.tensor(sel), nthreads=threads)
        done += n
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
        if time.perf_counter() - tb < 1.0:
            n *= 2
    elem = 2
    kvb, qb, ob, lb, ib = decode_bytes(B, Hq, w.Hkv, w.D, B * w.L, elem)
    step_bytes = kvb + qb + ob + lb + ib
    frac = done / len(rows_all)
    return dict(value=step_bytes * frac / el / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{done} of the {len(rows_all)} (request, query head) rows of the decode "
                       f"workload ({frac:.2f} steps) in {el:.1f} s, fp64 two-pass, OpenMP "
                       f"{threads} threads; GB/s = the same algorithmic bytes per row as the GPU")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import reduction_attention_amd as ra
    import synth
    ra._lib.load()
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream, args.warm_seconds)
    log(f"device: {torch.cuda.get_device_name(0)}, CUs: {ra.attn_device_cu_count()}")

    if args.only:
        fn = {"decode": lambda: bench_decode(torch, ra, synth, "llama3_8b_decode_bf16", args, timer),
              "ragged": lambda: bench_decode(torch, ra, synth, "ragged_decode_bf16", args, timer, 1),
              "ragged_flat": lambda: bench_decode_flat(torch, ra, synth, "ragged_decode_bf16",
                                                       args, timer),
              "prefill": lambda: bench_prefill(torch, ra, synth, args, timer),
              "bsr": lambda: bench_bsr(torch, ra, synth, args, timer),
              "bsr_heads": lambda: bench_bsr(torch, ra, synth, args, timer,
                                             "bsr_heads_prefill_fp16"),
              "append": lambda: bench_append(torch, ra, synth, args, timer),
              "mla": lambda: bench_mla(torch, ra, synth, "mla_decode_bf16", args, timer),
              "mla_ragged": lambda: bench_mla(torch, ra, synth, "mla_ragged_decode_bf16", args,
                                              timer),
              "copy": lambda: bench_copy(torch, args, timer)}[args.only]
        r = fn()
        print(json.dumps({"only": args.only, **r}))
        return

    d = bench_decode(torch, ra, synth, "llama3_8b_decode_bf16", args, timer)
    log(f"decode: {d['step_ms']*1e3:.1f} us/step, {d['gbs']:.0f} GB/s, s={d['splits']}; "
        f"partial kernel {d['kernel_ms']*1e3:.1f} us, {d['kernel_gbs']:.0f} GB/s")
    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("kernel_source_hash") == source_hash():
            traffic = tj.get("decode_partial_bytes")
    except (OSError, ValueError):
        pass
    roofline = dict(bound="hbm", achieved=round(d["kernel_gbs"], 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(d["kernel_gbs"] / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel="rattn::decode_partial_mfma<rattn::BF16, 128, 4, 1>",
                    algorithmic_bytes=d["kernel_bytes"],
                    avg_launch_us=round(d["kernel_ms"] * 1e3, 2))
    out = {
        "metric": METRIC,
        "value": round(d["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": d["workload"], "batch": d["B"], "q_heads": d["Hq"],
                   "kv_heads": d["Hkv"], "head_dim": d["D"], "kv_len": d["max_kv_len"],
                   "splits": d["splits"], "chunk": d["chunk"], "parallelism": "single-gpu",
                   "kv_copies_rotated": d["kv_copies_rotated"]},
        "roofline": roofline,
        "frac_of_hbm_peak": round(d["gbs"] / HBM_PEAK_GBS, 4),
    }
    if d["graph_step_ms"]:
        gb = d["step_bytes"] / d["graph_step_ms"] / 1e6
        out["graph_replay"] = dict(ms_per_step=round(d["graph_step_ms"], 5), gbs=round(gb, 1),
                                   frac=round(gb / HBM_PEAK_GBS, 4),
                                   note="the same step, ten per HIP graph replay")
        log(f"decode in HIP graphs: {d['graph_step_ms']*1e3:.1f} us/step, {gb:.0f} GB/s")
    if not args.no_also:
        also = {}
        p = bench_prefill(torch, ra, synth, args, timer)
        log(f"prefill: {p['ms']*1e3:.1f} us, {p['tflops']:.1f} TFLOP/s ({100*p['frac']:.1f}% of peak)")
        also["causal_prefill"] = dict(workload=p["workload"], ms=round(p["ms"], 4),
                                      tflops=round(p["tflops"], 1), frac=round(p["frac"], 4),
                                      roofline=dict(bound="mfma", achieved=round(p["tflops"], 1),
                                                    peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                                                    frac=round(p["frac"], 4),
                                                    algorithmic_flops=p["flops"]))
        r = bench_decode(torch, ra, synth, "ragged_decode_bf16", args, timer, rotate=1)
        rf = bench_decode_flat(torch, ra, synth, "ragged_decode_bf16", args, timer)
        log(f"ragged decode: flat plan {rf['step_ms']*1e3:.1f} us, {rf['gbs']:.0f} GB/s, "
            f"P={rf['pieces']}; chunk plan {r['step_ms']*1e3:.1f} us, {r['gbs']:.0f} GB/s, "
            f"s={r['splits']}")
        also["ragged_decode"] = dict(workload=r["workload"], plan="flat", ms=round(rf["step_ms"], 4),
                                     gbs=round(rf["gbs"], 1),
                                     frac=round(rf["gbs"] / HBM_PEAK_GBS, 4),
                                     total_kv=r["total_kv"], pieces=rf["pieces"],
                                     piece_len=rf["piece_len"], kv_bytes=r["kv_bytes"],
                                     chunk_plan=dict(ms=round(r["step_ms"], 4),
                                                     gbs=round(r["gbs"], 1), splits=r["splits"]))
        ap = bench_append(torch, ra, synth, args, timer)
        log(f"append prefill: {ap['ms']*1e3:.1f} us, {ap['tflops']:.1f} TFLOP/s, s={ap['splits']} "
            f"(unsplit {ap['ms_unsplit']*1e3:.1f} us)")
        also["append_prefill"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                  for k, v in ap.items()}
        for name, key in (("mla_decode_bf16", "mla_decode"),
                          ("mla_ragged_decode_bf16", "mla_ragged_decode")):
            m = bench_mla(torch, ra, synth, name, args, timer)
            log(f"{name}: {m['ms']*1e3:.1f} us, {m['gbs']:.0f} GB/s, s={m['splits']}, "
                f"{m['tflops']:.1f} TFLOP/s")
            also[key] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()}
        b = bench_bsr(torch, ra, synth, args, timer)
        log(f"bsr: {b['ms']*1e3:.1f} us ({b['kernel']}-wise; block {b['ms_block']*1e3:.1f}, "
            f"row {b['ms_row']*1e3:.1f}), {b['tflops_ot']:.1f} TFLOP/s at OT granularity")
        also["bsr_prefill"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in b.items()}
        bh = bench_bsr(torch, ra, synth, args, timer, "bsr_heads_prefill_fp16")
        log(f"bsr per-head-group masks, L {bh['L']}: {bh['ms']*1e3:.1f} us ({bh['kernel']}-wise; "
            f"block {bh['ms_block']*1e3:.1f}, row {bh['ms_row']*1e3:.1f})")
        also["bsr_heads_prefill"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                     for k, v in bh.items()}
        out["also"] = also
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(torch, synth, args.cpu_seconds)
        log(f"cpu baseline: {out['cpu_baseline']['value']:.3f} GB/s on "
            f"{out['cpu_baseline']['cores']} threads")
    print(json.dumps(out))


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "device.hpp"):
        with open(os.path.join(ROOT, "reduction_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
