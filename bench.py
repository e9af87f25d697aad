#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention path on one MI355X.

A step is one decode step of a 28-layer Qwen3-0.6B-shaped model at
concurrency 64: for each layer, store the 64 new tokens' K/V and run decode
attention over the paged cache, in one launch per layer (paged_decode_store;
`--unfused` runs kv_store + paged_decode instead).  Workload: 64 seqs, context U{512..1024}, block 256,
16 q heads / 8 KV heads / head_dim 128, bf16, 28 independent layer caches
(7 GiB), q pre-scaled.  Inputs are synthetic, drawn with fixed seeds, resident
in HBM before timing starts.  By default the step is captured once in a HIP
graph and replayed (the pages' decode runs with graph replay); the eager rate
is reported next to it.

Further legs, each timed alone: the varlen prefill over a cached prefix (16
seqs, new U{64..512}, prefix 0-2 blocks; MFMA utilisation; also fused with the
new tokens' store), the long-context decode (64 seqs, context U{4096..8192},
with and without a 256-token window; HBM fraction), the two small decode
workloads (latency), a mixed batch (48 decode rows + 4 prefill chunks, as one
varlen prefill and split by kind in one launch) and the 28-layer step at
context 512 for c = 1, 8 and 64, eager against graph replay (`--no-sweep`
skips it; `--no-legs` skips every leg).

Prints ONE JSON line.  `value` = algorithmic bytes of the step (K/V read by
decode for the admitted positions, q, out, block tables, kv_store traffic) /
step time, in GB/s.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "paged-decode KV GB/s (% HBM peak) + attn tokens/s at c=64; prefill MFMA %"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy_) three times: the "
                         "known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def decode_bytes(ctx, bs, hq, hkv, d, window=0):
    """Algorithmic bytes of one decode call: K and V rows of every admitted
    position, q, out, the used block-table entries and the context lengths."""
    kv = 0
    tbl = 0
    for L in ctx:
        L = int(L)
        lo = max(0, L - window) if window else 0
        kv += (L - lo) * hkv * d * 2 * 2
        tbl += (math.ceil(L / bs) - lo // bs) * 4 if L > 0 else 0
    n = len(ctx)
    return kv + 2 * n * hq * d * 2 + tbl + 4 * n


def store_bytes(n, hkv, d):
    return n * hkv * d * 2 * 2 * 2 + 4 * n


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode_and_prefill.md")
CSRC = os.path.join(ROOT, "paged_kv_cache_236_amd", "csrc")


def sources_digest(kernel_source: str) -> str:
    """sha256 (first 16 hex digits) of a kernel's sources: its launcher and
    kernel header, then device_common.h, launch.h and api.hip."""
    import hashlib
    m = hashlib.sha256()
    kernel_header = {"paged_decode.hip": "decode_kernel.h",
                     "paged_prefill.hip": "prefill_kernel.h"}[kernel_source]
    for f in (kernel_source, kernel_header, "device_common.h", "launch.h", "api.hip"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()[:16]


def profiled_traffic(record: str, kernel_source: str):
    """HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counter runs kept
    in profiles/ (each counter scaled by the factor the same counter reads for
    a plain copy of known size, recorded with the counters), or None when the
    kernel's sources changed since the counters were taken."""
    digest = sources_digest(kernel_source)
    try:
        with open(TRAFFIC_PROFILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    for line in lines:
        if not line.startswith("traffic-record:"):
            continue
        fields = dict(f.split("=", 1) for f in line.split()[2:])
        if line.split()[1] == record and fields.get("sources") == digest:
            fs = float(fields.get("fetch_scale", 2.0))
            ws = float(fields.get("write_scale", 1.0))
            return int(round((float(fields["fetch_kib"]) * fs + float(fields["write_kib"]) * ws)
                             * 1024))
    return None


def prefill_flops(lq, lk, hq, d, window=0):
    """4*d flops (QK^T and PV) per admitted (query, key) pair per q head."""
    pairs = 0
    for q_len, k_len in zip((int(v) for v in lq), (int(v) for v in lk)):
        p = k_len - q_len
        for i in range(q_len):
            t = p + i
            lo = max(0, t - window + 1) if window else 0
            pairs += t - lo + 1
    return int(4 * d * pairs * hq)


def copy_calibration():
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB), three times."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}); attention shards by KV head with no "
              f"exchange, so the per-GPU figure at N=1 is the one to read.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_236_amd as pk
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    nl = args.layers
    hq, hkv, d, bs = W.NUM_Q_HEADS, W.NUM_KV_HEADS, W.HEAD_DIM, 256

    # ---- inputs, resident before timing -------------------------------------
    layers = []
    for l in range(nl):
        meta = W.deep_decode_layer_meta(l)
        t = W.to_torch(meta, dev)
        t["k_cache"], t["v_cache"] = W.device_caches(W.DEEP_DECODE, 256, bs, dev, layer=l)
        t["out"] = torch.empty_like(t["q"])
        layers.append(t)
    ctx = meta.context_lens
    maxctx = int(ctx.max())
    scale = meta.scale
    ps, nparts = pk.decode_plan(64, hkv, maxctx)
    ws_bytes = pk.decode_workspace_size(64, hq, hkv, d, maxctx)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def store(t):
        pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])

    def decode(t):
        pk.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                        scale, max_context_len=maxctx, out=t["out"], workspace=ws)

    def fused(t):
        pk.paged_decode_store(t["q"], t["key"], t["value"], t["k_cache"], t["v_cache"],
                              t["block_tables"], t["context_lens"], scale, max_context_len=maxctx,
                              out=t["out"], workspace=ws)

    def step():
        for t in layers:
            if args.unfused:
                store(t)
                decode(t)
            else:
                fused(t)

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall / steps * 1e3

    for _ in range(args.warmup):
        step()
    eager_ms, eager_wall_ms = timed(step, args.steps)

    graph = None
    if args.mode == "graph":
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        graph_ms, graph_wall_ms = timed(graph.replay, args.steps)
        ms_per_step = max(graph_ms, graph_wall_ms)
    else:
        ms_per_step = max(eager_ms, eager_wall_ms)

    # ---- average launch duration of each call (events on its stream) ---------
    def per_call_us(fn, passes=5):
        # One launch per layer, back to back between one pair of events on the
        # launch stream; a spin kernel first gives the host a head start, so
        # the events time GPU work, not host launch gaps.  Mean over `passes`
        # passes of all layers (and the fastest pass).
        runs = []
        for _ in range(passes):
            torch.cuda.synchronize()
            torch.cuda._sleep(20_000_000)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for t in layers:
                fn(t)
            e1.record(stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) / len(layers) * 1e3)
        return sum(runs) / len(runs), min(runs)

    fused_us, fused_min_us = per_call_us(fused)
    dec_us, _ = per_call_us(decode)
    store_us, _ = per_call_us(store)

    dbytes = decode_bytes(ctx, bs, hq, hkv, d)
    sbytes = store_bytes(64, hkv, d)
    step_bytes = nl * (dbytes + sbytes)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    launch_us = dec_us if args.unfused else fused_us
    launch_bytes = dbytes if args.unfused else dbytes + sbytes
    dec_gbs = launch_bytes / (launch_us * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("decode step, 28 layers x (kv_store + paged_decode), c=64" if args.unfused
                         else "decode step, 28 layers x paged_decode_store (store + attend), c=64"),
            "num_seqs": 64, "context_lens": "U{512..1024}", "block_size": bs,
            "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d, "layers": nl,
            "mode": args.mode, "partition_size": ps, "partitions_per_seq": nparts,
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "attn_tokens_per_s": round(64 / (ms_per_step * 1e-3), 1),
        "eager_ms_per_step": round(max(eager_ms, eager_wall_ms), 4),
        "roofline": {
            "kernel": (("decode_partition_kernel" if nparts == 1 else "decode_partition_merged_kernel")
                       + ("" if args.unfused else " (fused store)")),
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": (profiled_traffic("decode_c64_fused", "paged_decode.hip")
                        if not args.unfused else None),
            "bytes_per_launch": launch_bytes,
            "us_per_launch": round(launch_us, 2),
            "us_per_launch_timing": "mean of 5 passes of 28 back-to-back launches (HIP events "
                                    "on the launch stream)",
            "fastest_pass_us": round(fused_min_us, 2) if not args.unfused else None,
        },
        "sources": {"decode": sources_digest("paged_decode.hip"),
                    "prefill": sources_digest("paged_prefill.hip")},
        "unfused": {"paged_decode_us": round(dec_us, 2), "kv_store_us": round(store_us, 2),
                    "paged_decode_GBps": round(dbytes / (dec_us * 1e-6) / 1e9, 1),
                    "kv_store_GBps": round(sbytes / (store_us * 1e-6) / 1e9, 1)},
    }

    # ---- prefill leg ----------------------------------------------------------
    if not args.no_prefill:
        try:
            result["prefill"] = prefill_leg(args, pk, W, dev, stream)
        except pk.PagedKVError as e:
            result["prefill"] = {"error": str(e)}

    if not args.no_legs:
        del layers
        if not args.no_sweep:
            result["graph_sweep"] = graph_sweep_leg(args, pk, W, dev, stream)
        result["long_decode"] = long_leg(args, pk, W, dev, stream)
        result["small_decode"] = small_leg(args, pk, W, dev, stream)
        result["mixed_batch"] = mixed_leg(args, pk, W, dev, stream)

    # ---- CPU baseline: the oracle on a bounded sample -------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W, dbytes)

    print(json.dumps(result), flush=True)


def time_call(fn, stream, n):
    import torch
    fn()
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


_FLUSH = {}


def time_cold(fn, stream, n):
    """Median time of n single launches, each after writing a 512 MiB buffer
    (twice the 256 MB MALL), so the launch finds none of its inputs cached."""
    import torch
    buf = _FLUSH.get("buf")
    if buf is None:
        buf = _FLUSH["buf"] = torch.empty(512 << 20, dtype=torch.uint8, device=torch.device("cuda:0"))
    fn()
    times = []
    for _ in range(n):
        buf.zero_()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return times[len(times) // 2]


def graph_sweep_leg(args, pk, W, dev, stream, concurrencies=(1, 8, 64), ctx=512, nl=28):
    """The 28-layer decode step (store + attend per layer, paged_decode_store)
    at c = 1, 8 and 64 sequences of context 512, eager against graph replay:
    where launch overhead, not HBM, sets the step time at small c.  Each mode
    is the median of three timed runs of max(steps, 20) steps."""
    import torch
    res = {"workload": f"decode step, {nl} layers x paged_decode_store, context {ctx} "
                       "(incl. the new token), block 256, 16/8/128 bf16",
           "pages_context_only": "the pages quote 80.24 tok/s eager and 242.64 tok/s graph replay "
                                 "at c=1 for a whole 351.6M model on other hardware; not a target"}
    bs = 256
    per_seq = (ctx + bs - 1) // bs
    for c in concurrencies:
        rng = W.rng_for(W.DEEP_DECODE, 1000 + c)
        tables = torch.from_numpy(
            rng.permutation(c * per_seq).astype("int32").reshape(c, per_seq)).to(dev)
        lens = torch.full((c,), ctx, dtype=torch.int32, device=dev)
        layers = []
        for l in range(nl):
            kc, vc = W.device_caches(W.DEEP_DECODE, c * per_seq, bs, dev, layer=1000 * c + l)
            q = W.device_normal_bf16((c, 16, 128), [W.DEEP_DECODE, 2000 + c, l], dev)
            kn = W.device_normal_bf16((c, 8, 128), [W.DEEP_DECODE, 3000 + c, l], dev)
            vn = W.device_normal_bf16((c, 8, 128), [W.DEEP_DECODE, 4000 + c, l], dev)
            layers.append((q, kn, vn, kc, vc, torch.empty_like(q)))
        ws_bytes = pk.decode_workspace_size(c, 16, 8, 128, ctx)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def step():
            for q, kn, vn, kc, vc, out in layers:
                pk.paged_decode_store(q, kn, vn, kc, vc, tables, lens, 1 / math.sqrt(128),
                                      max_context_len=ctx, out=out, workspace=ws)

        def timed(fn, n, reps=3):
            # Median of `reps` timed runs of n steps each: an eager step is host-bound at
            # small c, and a single host stall (tens of ms) would otherwise decide it.
            fn()
            torch.cuda.synchronize()
            runs = []
            for _ in range(reps):
                t0 = time.perf_counter()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(n):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                runs.append(max(e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3) / n * 1e3)
            return sorted(runs)[len(runs) // 2]

        n = max(args.steps, 20)
        eager_us = timed(step, n)
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        graph_us = timed(g.replay, n)
        res[f"c{c}"] = {"eager_us_per_step": round(eager_us, 1),
                        "graph_us_per_step": round(graph_us, 1),
                        "eager_tok_per_s": round(c / (eager_us * 1e-6), 1),
                        "graph_tok_per_s": round(c / (graph_us * 1e-6), 1),
                        "graph_speedup": round(eager_us / graph_us, 2)}
        del g, layers
        torch.cuda.synchronize()
    return res


def long_leg(args, pk, W, dev, stream):
    """64 seqs, context U{4096..8192}, block 256, 2 GiB cache: full and window 256."""
    import torch
    res = {}
    kc, vc = W.long_decode_device_caches(dev)
    for window in (0, 256):
        m = W.long_decode_meta(window)
        t = W.to_torch(m, dev)
        mcl = int(m.context_lens.max())
        out = torch.empty_like(t["q"])
        ps, nparts = pk.decode_plan(64, 8, mcl, window)

        def run():
            pk.paged_decode(t["q"], kc, vc, t["block_tables"], t["context_lens"], m.scale,
                            sliding_window=window, max_context_len=mcl, out=out)
        us = time_call(run, stream, 10)
        nbytes = decode_bytes(m.context_lens, 256, 16, 8, 128, window)
        gbs = nbytes / (us * 1e-6) / 1e9
        res["window_256" if window else "full"] = {
            "us_per_launch": round(us, 2), "bytes_per_launch": nbytes, "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "partition_size": ps, "partitions_per_seq": nparts}
        if window:
            # 67 MB fit the MALL when launches repeat; cold: flushed before each.
            us_cold = time_cold(run, stream, 11)
            res["window_256"]["cold_us_per_launch"] = round(us_cold, 2)
            res["window_256"]["cold_hbm_frac"] = round(nbytes / (us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    return res


def small_leg(args, pk, W, dev, stream):
    """8 seqs block 16 (decode), and 16 seqs block 256 (store + decode in one launch)."""
    import torch
    res = {}
    x = W.small_decode()
    t = W.to_torch(x, dev)
    mcl = x.max_context_len
    us = time_call(lambda: pk.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                           t["context_lens"], x.scale, max_context_len=mcl),
                   stream, 50)
    res["8seq_block16"] = {"us_per_launch": round(us, 2),
                           "bytes_per_launch": decode_bytes(x.context_lens, 16, 16, 8, 128)}
    y = W.store_decode()
    t = W.to_torch(y, dev)
    mcl = y.max_context_len
    us = time_call(lambda: pk.paged_decode_store(t["q"], t["key"], t["value"], t["k_cache"],
                                                 t["v_cache"], t["block_tables"], t["context_lens"],
                                                 y.scale, max_context_len=mcl), stream, 50)
    run_store = lambda: pk.paged_decode_store(t["q"], t["key"], t["value"], t["k_cache"],
                                              t["v_cache"], t["block_tables"], t["context_lens"],
                                              y.scale, max_context_len=mcl)
    res["16seq_block256_store"] = {"us_per_launch": round(us, 2),
                                   "cold_us_per_launch": round(time_cold(run_store, stream, 11), 2),
                                   "bytes_per_launch": decode_bytes(y.context_lens, 256, 16, 8, 128)
                                   + store_bytes(16, 8, 128)}
    return res


def mixed_leg(args, pk, W, dev, stream):
    """A chunked-prefill step (48 decode sequences + 4 prefill chunks, 3255 query
    rows, block 256) in one varlen prefill launch."""
    import numpy as np
    import torch
    x = W.mixed_batch()
    t = W.to_torch(x, dev)
    lq = np.diff(x.cu_seqlens_q)
    lk = np.diff(x.cu_seqlens_k)
    msq = int(lq.max())
    out = torch.empty_like(t["q"])
    pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])

    def run():
        pk.paged_prefill(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["cu_seqlens_q"],
                         t["cu_seqlens_k"], x.scale, max_seqlen_q=msq, out=out)
    us = time_call(run, stream, 10)
    # The same step split by kind: the decode rows on the decode kernel, the
    # chunks on the prefill kernel (two launches).
    nd = int(np.sum(lq == 1))
    mdcl = int(lk[:nd].max())
    ws = torch.empty(max(pk.decode_workspace_size(nd, W.NUM_Q_HEADS, W.NUM_KV_HEADS, W.HEAD_DIM,
                                                  mdcl), 1), dtype=torch.uint8, device=dev)

    def run_split():
        pk.paged_prefill_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                t["cu_seqlens_q"], t["cu_seqlens_k"], x.scale, num_decode_seqs=nd,
                                max_seqlen_q=int(lq[nd:].max()), max_decode_context_len=mdcl,
                                out=out, workspace=ws)
    us_split = time_call(run_split, stream, 10)
    flops = prefill_flops(lq, lk, W.NUM_Q_HEADS, W.HEAD_DIM)
    kv_bytes = int(lk.sum()) * W.NUM_KV_HEADS * W.HEAD_DIM * 2 * 2
    return {"workload": "chunked-prefill step: 48 decode seqs (ctx U{256..2048}) + 4 prefill chunks "
                        "(U{256..1024} new over 0-4 blocks), 4096-token budget",
            "split_by_kind_us": round(us_split, 2),
            "total_q": int(lq.sum()), "us_per_launch": round(us, 2), "flops_per_launch": flops,
            "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 2),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kv_bytes_once": kv_bytes, "kv_GB/s": round(kv_bytes / (us * 1e-6) / 1e9, 1)}


def prefill_leg(args, pk, W, dev, stream):
    import numpy as np
    import torch
    x = W.prefix_prefill()
    t = W.to_torch(x, dev)
    lq = np.diff(x.cu_seqlens_q)
    lk = np.diff(x.cu_seqlens_k)
    msq = int(lq.max())
    out = torch.empty_like(t["q"])

    def run():
        pk.paged_prefill(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["cu_seqlens_q"],
                         t["cu_seqlens_k"], x.scale, max_seqlen_q=msq, out=out)

    pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    n = max(args.steps, 10)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    flops = prefill_flops(lq, lk, W.NUM_Q_HEADS, W.HEAD_DIM)
    tflops = flops / (us * 1e-6) / 1e12

    # The step with the new tokens' store: separate kv_store + prefill, and the
    # fused entry (one launch; it rewrites the same values each time).
    def unfused():
        pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
        run()

    def fused():
        pk.paged_prefill_store(t["q"], t["key"], t["value"], t["k_cache"], t["v_cache"],
                               t["block_tables"], t["cu_seqlens_q"], t["cu_seqlens_k"], x.scale,
                               max_seqlen_q=msq, out=out)
    us_unfused = time_call(unfused, stream, n)
    us_fused = time_call(fused, stream, n)
    us_store = time_call(lambda: pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"],
                                             t["v_cache"]), stream, n)
    sb = store_bytes(int(lq.sum()), W.NUM_KV_HEADS, W.HEAD_DIM)
    return {
        "workload": "varlen causal prefill, 16 seqs, new U{64..512}, prefix 0-2 x 256",
        "total_q": int(lq.sum()), "us_per_launch": round(us, 2), "flops_per_launch": flops,
        "store_then_prefill_us": round(us_unfused, 2), "fused_store_prefill_us": round(us_fused, 2),
        "kv_store_us": round(us_store, 2), "kv_store_GBps": round(sb / (us_store * 1e-6) / 1e9, 1),
        "roofline": {"kernel": "paged_prefill_kernel", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": profiled_traffic("prefill_prefix", "paged_prefill.hip")},
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(W, dbytes_per_layer, sample_layers=4, layers_per_step=28, reps=3):
    """The oracle, untuned, on the host's cores: decode layers of the same
    28-layer workload (64 seqs, all 16 heads).  Drawing a layer's 268 MB of
    caches costs more than attending over it, so a sample of `sample_layers`
    of the 28 layers is drawn (outside the timing); one untimed warmup pass
    over the sample, then the median of `reps` timed passes, scaled to the
    28-layer step.  NumPy's BLAS gets one thread per core of the process's
    CPU affinity."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    blas_threads = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limits = threadpool_limits(cores)
        blas_threads = sorted({int(i.get("num_threads", 0)) for i in threadpool_info()}) or None
    except Exception:
        limits = None
    inputs = []
    for layer in range(sample_layers):
        x = W.deep_decode_layer(layer)
        kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
        inputs.append((x, kc, vc))

    def one_pass():
        t0 = time.perf_counter()
        for x, kc, vc in inputs:
            oracle.paged_decode(x.q, kc, vc, x.block_tables, x.context_lens, x.scale)
        return time.perf_counter() - t0

    one_pass()                                   # warmup
    times = sorted(one_pass() for _ in range(reps))
    med = times[len(times) // 2]
    per_layer = med / sample_layers
    if limits is not None and hasattr(limits, "unregister"):
        limits.unregister()
    gbs = dbytes_per_layer / per_layer / 1e9
    step_s = per_layer * layers_per_step
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample_layers} of the {layers_per_step} decode layers (64 seqs x 16 heads, "
                      f"ctx U{{512..1024}}), 1 warmup + median of {reps} passes over them "
                      f"({med:.2f} s per pass), scaled to the {layers_per_step}-layer step; "
                      "float64 NumPy oracle",
            "ms_per_step_equiv": round(step_s * 1e3, 1),
            "attn_tokens_per_s_equiv": round(64 / step_s, 3),
            "blas_threads": blas_threads,
            "cpu": cpu_model()}


if __name__ == "__main__":
    main()
