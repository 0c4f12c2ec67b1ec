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
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--splits", type=int, default=0, help="force the decode split count")
    p.add_argument("--only", choices=["decode", "prefill", "ragged", "ragged_flat", "mla",
                                      "mla_ragged", "bsr", "bsr_window", "bsr_cols", "bsr_heads",
                                      "bsr_long",
                                      "append", "tiny", "sweep", "copy"],
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


def pct(x, q):
    """The q-quantile of x (nearest rank)."""
    s = sorted(x)
    return s[min(len(s) - 1, int(q * len(s)))]


def spread(ms):
    """p10 / p90 of per-step times in ms (rounded)."""
    return dict(ms_p10=round(pct(ms, 0.1), 5), ms_p90=round(pct(ms, 0.9), 5))


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
                step_ms=step_ms, step_ms_p10=pct(ms, 0.1), step_ms_p90=pct(ms, 0.9),
                step_bytes=step_bytes, o=o, lse=lse,
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
                gbs=(kvb + qb + ob + lb + ib) / t / 1e6, **spread(ms))


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
    wide = w.Hq >= 64 and w.Hq % 64 == 0
    kernel = "mla_wide_kernel" if wide else "mla_decode_kernel"
    out = dict(workload=wname, B=w.B, H=w.Hq, total_kv=total, max_kv_len=max_len, plan="chunk",
               splits=s, kernel=kernel, ms=t, **spread(ms), bytes=byt, gbs=byt / t / 1e6,
               frac=byt / t / 1e6 / HBM_PEAK_GBS, tflops=flops / t / 1e9,
               frac_mfma=flops / t / 1e9 / MFMA_BF16_PEAK_TFS)
    if wide and max_len * w.B != total:
        # ragged many-head batch: also time the flat plan (equal pieces of
        # the packed cache) beside the chunk plan
        P = ra.attn_mla_decode_flat_pieces(w.B, w.Hq, total)
        wsf = torch.empty(max(ra.attn_mla_decode_flat_workspace_bytes(w.B, w.Hq, max_len, total, P),
                              256), dtype=torch.uint8, device=q.device)
        msf, _ = timer.run(lambda i: ra.attn_mla_decode_flat(q, kv, kvp, max_len, w.scale,
                                                             num_pieces=P, o=o, lse=lse,
                                                             workspace=wsf, stream=stream),
                           args.steps, args.warmup)
        tf = median(msf)
        out["flat_plan"] = dict(pieces=P, piece_len=-(-total // P), ms=tf, gbs=byt / tf / 1e6,
                                tflops=flops / tf / 1e9)
    return out


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
                ms=t, **spread(ms), flops=flops, tflops=flops / t / 1e9,
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
                dtype="bf16", splits=s, ms=t, **spread(ms), flops=flops,
                tflops=flops / t / 1e9,
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
    times, spreads = {}, {}
    for kern in ("block", "row"):
        ms, _ = timer.run(lambda i: ra.attn_prefill_bsr(q, k, v, md, o=o, lse=lse, stream=stream,
                                                        kernel=kern), args.steps, args.warmup)
        times[kern] = median(ms)
        spreads[kern] = spread(ms)
    # every mask serves Hq / num_masks heads
    hpm = w.Hq // m.num_masks
    n_ot = m.nnz_full + m.nnz_part
    flops_ot = 4 * w.D * 64 * 64 * n_ot * hpm * w.B
    flops_rows = 4 * w.D * 16 * 16 * plan["row_blocks"] * hpm * w.B
    valid = int(inp["mask"].to(torch.int64).sum())
    flops_valid = 4 * w.D * valid * hpm * w.B
    t = times[plan["kernel"]]  # what kernel="auto" runs
    return dict(workload=w.name, B=w.B, L=w.L, H=w.Hq, D=w.D, dtype="fp16", ms=t,
                **spreads[plan["kernel"]],
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
    return dict(bytes_read=n, bytes_written=n, ms=median(ms), **spread(ms),
                gbs=2 * n / median(ms) / 1e6)


def bench_tiny_decode(torch, ra, synth, args, timer):
    """The tiny fp32 decode (1 request, 4/1 heads, D 64, 256 keys) at each of
    its split counts: launch-latency bound, microseconds per step."""
    w = synth.workload("tiny_decode_fp32")
    inp = w.make("cuda:0")
    q, k, v, kvp = inp["q"], inp["k"], inp["v"], inp["kv_indptr"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    out = {}
    for s in w.splits:
        ws = torch.empty(ra.attn_decode_workspace_bytes(w.B, w.Hq, w.D, s), dtype=torch.uint8,
                         device=q.device)
        ms, _ = timer.run(lambda i: ra.attn_decode_splitkv(q, k, v, kvp, w.L, num_splits=s, o=o,
                                                           lse=lse, workspace=ws, stream=stream),
                          args.steps, args.warmup)
        out[f"s{s}"] = dict(us=round(median(ms) * 1e3, 2), us_p10=round(pct(ms, 0.1) * 1e3, 2),
                            us_p90=round(pct(ms, 0.9) * 1e3, 2))
    return dict(workload=w.name, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, kv_len=w.L, dtype="fp32",
                **out)


def bench_split_sweep(torch, ra, synth, args, timer, splits=(1, 2, 4, 8, 16, 32, 64)):
    """The headline decode step at split counts 1 .. 64 (the rule picks 8)."""
    w = synth.workload("llama3_8b_decode_bf16")
    inp = w.make("cuda:0")
    q, kvp = inp["q"], inp["kv_indptr"]
    sets = [(inp["k"], inp["v"])] + [(inp["k"].clone(), inp["v"].clone()) for _ in range(2)]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    kvb, qb, ob, lb, ib = decode_bytes(w.B, w.Hq, w.Hkv, w.D, w.B * w.L, 2)
    out = {}
    for s in splits:
        ws = torch.empty(max(ra.attn_decode_workspace_bytes(w.B, w.Hq, w.D, s), 256),
                         dtype=torch.uint8, device=q.device)

        def step(i):
            k, v = sets[i % 3]
            ra.attn_decode_splitkv(q, k, v, kvp, w.L, num_splits=s, o=o, lse=lse, workspace=ws,
                                   stream=stream)

        ms, _ = timer.run(step, args.steps, args.warmup)
        t = median(ms)
        out[f"s{s}"] = dict(chunk=-(-w.L // s), us=round(t * 1e3, 2),
                            gbs=round((kvb + qb + ob + lb + ib) / t / 1e6, 1))
    return out


def cpu_threads():
    """Threads the oracle runs on: OMP_NUM_THREADS when it is set (the share
    of the host's CPUs that goes with one GPU), else every CPU this process
    may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    aff = len(os.sched_getaffinity(0))
    return (int(env) if env.isdigit() and int(env) > 0 else aff), aff


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _grow(run, total, budget_s):
    """Run ``run(start, n)`` on growing batches of a fixed seeded row order
    until about budget_s seconds have passed; returns (rows done, seconds)."""
    n, pos, t0 = 8, 0, time.perf_counter()
    while True:
        tb = time.perf_counter()
        run(pos, n)
        pos += n
        el = time.perf_counter() - t0
        if el >= budget_s or pos >= total:
            return pos, el
        if time.perf_counter() - tb < 1.0:
            n *= 2
        n = min(n, total - pos)


def cpu_baseline(torch, synth, budget_s, gpu_decode=None):
    """The fp64 oracle, as it stands, on bounded samples of the workloads:
    the headline decode (about ``budget_s`` seconds) and, with a quarter of
    that each, the ragged decode, the causal prefill and the block-sparse
    prefill, each as a rate in its own unit plus the extrapolated wall time
    of one full oracle evaluation.  With ``gpu_decode`` = (o, lse) of the
    headline decode, the sampled rows are also compared with the GPU's."""
    import oracle
    threads, aff = cpu_threads()

    def host(inp):
        return {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in inp.items()}

    # -- headline decode: (request, query head) rows in order --------------
    w = synth.workload("llama3_8b_decode_bf16")
    inp = host(w.make("cuda:0"))
    B, Hq = w.B, w.Hq
    qo = list(range(B + 1))
    rows_all = torch.tensor([(b, h) for b in range(B) for h in range(Hq)], dtype=torch.int64)
    errs = []

    def run_decode(pos, n):
        sel = rows_all[torch.arange(pos, pos + n) % len(rows_all)]
        o_r, l_r = oracle.attention(inp["q"], inp["k"], inp["v"], qo, inp["kv_indptr"], w.scale,
                                    rows=sel, nthreads=threads)
        if gpu_decode is not None and pos < len(rows_all):
            keep = min(n, len(rows_all) - pos)
            og, lg = gpu_decode
            b, h = sel[:keep, 0], sel[:keep, 1]
            errs.append(((og[b, h].double() - o_r[:keep]).abs().max().item(),
                         (lg[b, h].double() - l_r[:keep]).abs().max().item(), keep))

    done, el = _grow(run_decode, 10 ** 9, budget_s)
    kvb, qb, ob, lb, ib = decode_bytes(B, Hq, w.Hkv, w.D, B * w.L, 2)
    step_bytes = kvb + qb + ob + lb + ib
    frac = done / len(rows_all)
    out = dict(value=step_bytes * frac / el / 1e9, unit="GB/s", cores=threads, kind="oracle",
               sample=f"{done} of the {len(rows_all)} (request, query head) rows of the decode "
                      f"workload ({frac:.2f} steps) in {el:.1f} s, fp64 two-pass, OpenMP "
                      f"{threads} threads; GB/s = the same algorithmic bytes per row as the GPU",
               host_cpus=aff, cpu_model=cpu_model(),
               threads_note="OpenMP threads = OMP_NUM_THREADS when set (the host's CPU share "
                            "for one GPU), else the process's CPU affinity count",
               full_eval_s_est=round(el / frac, 3))
    if errs:
        out["parity_sample"] = dict(rows=sum(e[2] for e in errs),
                                    max_abs_o=max(e[0] for e in errs),
                                    max_abs_lse=max(e[1] for e in errs))
    per = {"llama3_8b_decode_bf16": dict(value=round(out["value"], 3), unit="GB/s",
                                         full_eval_s_est=out["full_eval_s_est"])}
    sub = budget_s / 4
    g = torch.Generator().manual_seed(12345)

    # -- ragged decode: rows weighted by their request's length -------------
    w = synth.workload("ragged_decode_bf16")
    inp = host(w.make("cuda:0"))
    lens = inp["lengths"]
    order = torch.randperm(w.B * w.Hq, generator=g)
    rows = torch.stack([order // w.Hq, order % w.Hq], 1)
    work = 0

    def run_ragged(pos, n):
        nonlocal work
        sel = rows[pos:pos + n]
        oracle.attention(inp["q"], inp["k"], inp["v"], list(range(w.B + 1)), inp["kv_indptr"],
                         w.scale, rows=sel, nthreads=threads)
        work += sum(lens[int(b)] for b in sel[:, 0])

    done, el = _grow(run_ragged, len(rows), sub)
    frac = work / (w.Hq * sum(lens))
    kvb, qb, ob, lb, ib = decode_bytes(w.B, w.Hq, w.Hkv, w.D, sum(lens), 2)
    per[w.name] = dict(value=round((kvb + qb + ob + lb + ib) * frac / el / 1e9, 3), unit="GB/s",
                       rows=done, seconds=round(el, 2), full_eval_s_est=round(el / frac, 2))

    # -- causal prefill: FLOPs of the sampled rows' valid keys ---------------
    w = synth.workload("causal_prefill_bf16")
    inp = host(w.make("cuda:0"))
    order = torch.randperm(w.B * w.L * w.Hq, generator=g)
    rows = torch.stack([order // w.Hq, order % w.Hq], 1)
    flops = 0

    def run_prefill(pos, n):
        nonlocal flops
        sel = rows[pos:pos + n]
        oracle.attention(inp["q"], inp["k"], inp["v"], inp["qo_indptr"], inp["kv_indptr"],
                         w.scale, oracle.MASK_CAUSAL, rows=sel, nthreads=threads)
        flops += 4 * w.D * int(((sel[:, 0] % w.L) + 1).sum())

    done, el = _grow(run_prefill, len(rows), sub)
    total = causal_flops(w.B, w.Hq, w.L, w.D)
    per[w.name] = dict(value=round(flops / el / 1e9, 3), unit="GFLOP/s", rows=done,
                       seconds=round(el, 2), full_eval_s_est=round(el * total / flops, 1))

    # -- block-sparse prefill: FLOPs over the valid (query, key) pairs -------
    w = synth.workload("bsr_prefill_fp16")
    inp = host(w.make("cuda:0"))
    valid_per_row = inp["mask"].to(torch.int64).sum(1)
    order = torch.randperm(w.L * w.Hq, generator=g)
    rows = torch.stack([order // w.Hq, order % w.Hq], 1)
    flops = 0

    def run_bsr(pos, n):
        nonlocal flops
        sel = rows[pos:pos + n]
        oracle.attention(inp["q"][0], inp["k"][0], inp["v"][0], [0, w.L], [0, w.L], w.scale,
                         oracle.MASK_DENSE, inp["mask"], rows=sel, nthreads=threads)
        flops += 4 * w.D * int(valid_per_row[sel[:, 0]].sum())

    done, el = _grow(run_bsr, len(rows), sub)
    total = 4 * w.D * int(valid_per_row.sum()) * w.Hq
    per[w.name] = dict(value=round(flops / el / 1e9, 3), unit="GFLOP/s (valid pairs)",
                       rows=done, seconds=round(el, 2), full_eval_s_est=round(el * total / flops, 1))
    out["per_config"] = per
    return out


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
              "bsr_window": lambda: bench_bsr(torch, ra, synth, args, timer,
                                              "bsr_window_prefill_fp16"),
              "bsr_cols": lambda: bench_bsr(torch, ra, synth, args, timer,
                                            "bsr_cols_prefill_fp16"),
              "bsr_heads": lambda: bench_bsr(torch, ra, synth, args, timer,
                                             "bsr_heads_prefill_fp16"),
              "bsr_long": lambda: bench_bsr(torch, ra, synth, args, timer,
                                            "bsr_long_prefill_fp16"),
              "tiny": lambda: bench_tiny_decode(torch, ra, synth, args, timer),
              "sweep": lambda: bench_split_sweep(torch, ra, synth, args, timer),
              "append": lambda: bench_append(torch, ra, synth, args, timer),
              "mla": lambda: bench_mla(torch, ra, synth, "mla_decode_bf16", args, timer),
              "mla_ragged": lambda: bench_mla(torch, ra, synth, "mla_ragged_decode_bf16", args,
                                              timer),
              "copy": lambda: bench_copy(torch, args, timer)}[args.only]
        r = {k: v for k, v in fn().items() if k not in ("o", "lse")}
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
                    avg_launch_us=round(d["kernel_ms"] * 1e3, 2),
                    # the whole step (partial kernel + merge + the gap between
                    # them) against the same peak, on the step's algorithmic bytes
                    step_achieved=round(d["gbs"], 1), step_frac=round(d["gbs"] / HBM_PEAK_GBS, 4),
                    step_bytes=d["step_bytes"])
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
        "step_ms_p10": round(d["step_ms_p10"], 5),
        "step_ms_p90": round(d["step_ms_p90"], 5),
        "source_sha16": source_hash(all_sources=True),
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
                                      ms_p10=p["ms_p10"], ms_p90=p["ms_p90"],
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
                                     ms_p10=rf["ms_p10"], ms_p90=rf["ms_p90"],
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
            fp = m.get("flat_plan")
            log(f"{name}: {m['ms']*1e3:.1f} us, {m['gbs']:.0f} GB/s, s={m['splits']}, "
                f"{m['tflops']:.1f} TFLOP/s"
                + (f"; flat plan {fp['ms']*1e3:.1f} us, P={fp['pieces']}" if fp else ""))
            also[key] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()}
        for name, key in (("bsr_prefill_fp16", "bsr_prefill"),
                          ("bsr_window_prefill_fp16", "bsr_window_prefill"),
                          ("bsr_cols_prefill_fp16", "bsr_cols_prefill"),
                          ("bsr_heads_prefill_fp16", "bsr_heads_prefill"),
                          ("bsr_long_prefill_fp16", "bsr_long_prefill")):
            b = bench_bsr(torch, ra, synth, args, timer, name)
            log(f"{name}: L {b['L']}, {b['nnz_full'] + b['nnz_part']} stored OTs: "
                f"{b['ms']*1e3:.1f} us ({b['kernel']}-wise; block {b['ms_block']*1e3:.1f}, "
                f"row {b['ms_row']*1e3:.1f}), {b['tflops_ot']:.1f} TFLOP/s at OT granularity")
            also[key] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in b.items()}
        t = bench_tiny_decode(torch, ra, synth, args, timer)
        log(f"tiny fp32 decode: " + ", ".join(f"{k} {v['us']} us" for k, v in t.items()
                                              if k.startswith("s")))
        also["tiny_decode"] = t
        also["decode_split_sweep"] = bench_split_sweep(torch, ra, synth, args, timer)
        log("decode split sweep: " + ", ".join(f"{k} {v['us']} us"
                                               for k, v in also["decode_split_sweep"].items()))
        c = bench_copy(torch, args, timer)
        log(f"device copy (1 GiB): {c['gbs']:.0f} GB/s")
        also["copy"] = dict(bytes_read=c["bytes_read"], bytes_written=c["bytes_written"],
                            ms=round(c["ms"], 4), ms_p10=c["ms_p10"], ms_p90=c["ms_p90"],
                            gbs=round(c["gbs"], 1), frac=round(c["gbs"] / HBM_PEAK_GBS, 4),
                            note="torch device copy of 1 GiB: a measured reference for the "
                                 "HBM peak")
        out["also"] = also
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(torch, synth, args.cpu_seconds,
                                           gpu_decode=(d["o"].cpu(), d["lse"].cpu()))
        cb = out["cpu_baseline"]
        log(f"cpu baseline: {cb['value']:.3f} GB/s on {cb['cores']} threads ({cb['cpu_model']}); "
            + ", ".join(f"{k} {v['value']} {v['unit']}" for k, v in cb["per_config"].items()))
    print(json.dumps(out))


def source_hash(all_sources=False) -> str:
    """Hash of the decode kernel's sources (the key of the stored traffic
    counters), or of every library source and header (the record's source
    identity on a box without the repository's history)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "reduction_attention_amd", "csrc")
    files = [os.path.join(csrc, f) for f in ("decode.hip", "device.hpp")]
    if all_sources:
        files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                       if f.endswith((".hip", ".hpp", ".cpp")))
        files.append(os.path.join(ROOT, "include", "attn.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
