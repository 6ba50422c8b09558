#!/usr/bin/env python3
"""Benchmark PagedAttention V2 decode on one MI355X.

A step is one pass of the whole hot path over one batch: phase 1 (the
per-partition kernel) and phase 2 (the log-sum-exp combine), launched through
the C ABI on the current stream, on synthetic inputs already resident in HBM.

Default workload: 4 sequences x 100000 tokens, 24 query heads over 4 kv heads
(GQA 6), head size 256, bf16, block size 16 -- the long-context GQA decode the
metric names.  `--config` selects one of the other workloads.  `--entry v1`
times the single-pass entry point instead (one launch per step), `--entry
auto` whichever of the two the library's planner picks for the workload.

Prints ONE JSON line.  `value` is KV bytes read per second (decimal GB/s);
`roofline` reports phase 1's algorithmic bytes per launch over its mean
duration (HIP events on the launch stream, inside the timed region, on every
fifth step) against
MI355X's 8 TB/s HBM peak; `cpu_baseline` times the float64 CPU oracle on a
bounded sample of the same workload and also checks those outputs against the
GPU's.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0
EVENT_EVERY = 5      # timed steps per phase-1 event pair

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_attention_paged_v2_amd import workloads as W  # noqa: E402
from decode_attention_paged_v2_amd import accounting  # noqa: E402
import decode_attention_paged_v2_amd as pav2  # noqa: E402

DESCR = {
    "tiny": "1 seq x 1000 tokens, H=4, kv_h=4, d=64, fp32, block 16",
    "batched_gqa": "32 seqs, L~U[512,4096], H=32, kv_h=8, d=128, fp16, block 16",
    "long_gqa": "4 seqs x 100000 tokens, H=24, kv_h=4 (GQA 6), d=256, bf16, block 16",
    "ragged_alibi": "256 seqs, L log-uniform [1,32768] (4 empty), H=32, kv_h=8, d=80, fp16, ALiBi, block 16",
    "fp8_kv": "64 seqs x 16384 tokens, H=64, kv_h=8, d=128, e4m3 KV (k_scale 0.05, v_scale 0.04), bf16 q/out, block 32",
}
DTYPE_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def cpu_baseline(wl, out_gpu, target_core_seconds=15.0, max_threads=16):
    """Time the oracle on whole (seq, kv head) groups of the same workload."""
    import oracle
    gqa = wl.num_heads // wl.num_kv_heads
    groups = [(s, g) for s in range(wl.num_seqs) for g in range(wl.num_kv_heads)
              if wl.seq_lens_host[s] > 0]
    rng = np.random.default_rng(0)
    rng.shuffle(groups)
    # calibrate on one head, then take enough groups for ~target core-seconds
    s0, g0 = groups[0]
    host = wl.to("cpu")
    kw = dict(num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
              max_num_partitions=wl.max_num_partitions, q_dtype=oracle.dtype_code(wl.q_dtype),
              kv_dtype=oracle.dtype_code(wl.kv_dtype), alibi_slopes=host.alibi_slopes,
              k_scale=wl.k_scale, v_scale=wl.v_scale)
    args = (host.query, host.key_cache, host.value_cache, host.block_tables, host.seq_lens)
    t0 = time.perf_counter()
    oracle.paged_attention_v2(*args, pairs=[(s0, g0 * gqa)], threads=1, **kw)
    per_head = max(1e-3, time.perf_counter() - t0)
    n_groups = int(max(1, min(len(groups), round(target_core_seconds / (per_head * gqa)))))
    sample = groups[:n_groups]
    pairs = [(s, g * gqa + r) for s, g in sample for r in range(gqa)]
    threads = int(max(1, min(len(pairs), os.cpu_count() or 1, max_threads)))
    t0 = time.perf_counter()
    r = oracle.paged_attention_v2(*args, pairs=pairs, threads=threads, **kw)
    dt = time.perf_counter() - t0
    kvb = W.elem_size(wl.kv_dtype)
    bytes_ = sum(wl.seq_lens_host[s] * 2 * wl.head_size * kvb for s, g in sample)
    toks = sum(wl.seq_lens_host[s] for s, g in sample) * gqa
    err = 0.0
    for s, h in pairs:
        ref = torch.from_numpy(r["out"][s, h]).to(wl.q_dtype).double()
        err = max(err, float((out_gpu[s, h].double() - ref).abs().max()))
    return {
        "value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"{n_groups} of {len(groups)} (seq, kv head) groups = {len(pairs)} query heads, "
                   f"{bytes_ / 1e6:.1f} MB of KV, float64 C oracle, {dt:.2f} s wall"),
        "tokens_heads_per_s": round(toks / dt, 1),
        "seconds": round(dt, 3),
        "parity_max_abs_err_vs_gpu": err,
    }


def measured_traffic(config, entry="v2"):
    """HBM bytes per phase-1 launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain
    copy's reading) from the committed counter summary, or None when there is
    none or it was taken on different kernel sources."""
    from decode_attention_paged_v2_amd import rocprof_harness
    name = f"phase1_{config}.json" if entry == "v2" else f"v1_{config}.json"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    if data.get("source_hash") != rocprof_harness.source_hash() or "phase1_traffic_bytes" not in data:
        return None
    return round(float(data["phase1_traffic_bytes"]))


def _time_launches(fn, steps, warmup, stream):
    """Mean / min event time (ms) of fn() launches on `stream`, and wall ms per launch."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    return float(np.mean(ms)), float(np.min(ms)), wall


def cache_write_cpu_baseline(wl, target_core_seconds=10.0):
    """The oracle's cache write on a bounded sample of the workload's tokens (one thread)."""
    import oracle
    T = wl.key.shape[0]
    kvh, d = wl.key.shape[1], wl.key.shape[2]
    bs = wl.value_cache.shape[3]
    code = oracle.dtype_code(wl.cache_dtype)

    def run(n):
        k, v = wl.key[:n].cpu(), wl.value[:n].cpu()
        nb = (n + bs - 1) // bs
        kc = torch.empty((nb,) + tuple(wl.key_cache.shape[1:]), dtype=wl.key_cache.dtype)
        vc = torch.empty((nb,) + tuple(wl.value_cache.shape[1:]), dtype=wl.value_cache.dtype)
        t0 = time.perf_counter()
        oracle.reshape_and_cache(k, v, kc, vc, torch.arange(n), block_size=bs, cache_dtype=code,
                                 k_scale=wl.k_scale, v_scale=wl.v_scale)
        return time.perf_counter() - t0
    n0 = min(T, 256)
    per_tok = max(1e-7, run(n0) / n0)
    n = int(max(1, min(T, target_core_seconds / per_tok)))
    dt = run(n)
    bytes_ = n * kvh * d * 2 * (wl.key.element_size() + wl.key_cache.element_size())
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {T} tokens ({bytes_ / 1e6:.1f} MB moved), C oracle, {dt:.2f} s wall",
            "seconds": round(dt, 3)}


def cache_write_bench(args, dev):
    """KV-cache write: the whole context of the workload as one launch (the
    prefill of every sequence), and the decode step's one token per sequence."""
    pav2.load()
    spec = W.SPECS[args.config]
    stream = torch.cuda.current_stream(dev)
    res = {}
    for kind in ("prefill", "decode_step"):
        wl = W.cache_write_workload(spec, dev, decode_step=kind == "decode_step")
        kvdt = "fp8_e4m3" if wl.cache_dtype == torch.float8_e4m3fn else "auto"
        fn = lambda: pav2.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, wl.slot_mapping,
                                            kvdt, wl.k_scale, wl.v_scale)
        mean, mn, wall = _time_launches(fn, args.steps, args.warmup, stream)
        res[kind] = {"tokens": int(wl.key.shape[0]), "bytes_moved": wl.bytes_moved(),
                     "ms_mean": round(mean, 5), "ms_min": round(mn, 5), "wall_ms_per_launch": round(wall, 5),
                     "GBps": round(wl.bytes_moved() / (mean * 1e-3) / 1e9, 2)}
        if kind == "prefill":
            big = wl
        else:
            del wl
    p = res["prefill"]
    achieved = p["bytes_moved"] / (p["ms_mean"] * 1e-3) / 1e9
    result = {
        "metric": "KV-cache write GB/s (input read + cache written) and % of HBM peak",
        "value": round(achieved, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": p["ms_mean"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[big.key.dtype] + ("->fp8_e4m3" if big.cache_dtype == torch.float8_e4m3fn else ""),
        "data": "synthetic",
        "config": {"workload": f"{args.config} context written through its block tables: {DESCR[args.config]}",
                   "tokens": p["tokens"]},
        "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "prefill": p, "decode_step": res["decode_step"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_cache_traffic(args.config),
                     "kernel": "cache_write_kernel", "algorithmic_bytes_per_launch": p["bytes_moved"]},
        "library": pav2.lib_path(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cache_write_cpu_baseline(big)
    return result


# Block-sparse decode benchmark pattern on the long-context workload:
# (tp_rank, local_blocks, vert_stride, sparse block size, head sliding step)
# -- 64-token sparse blocks, the last 16 of them (1024 tokens) as the local
# window, and every 8th block, the same stripes for every head.
BLOCKSPARSE_PATTERN = (0, 16, 8, 64, 0)

MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFIX_CASE = dict(ctx=[16384] * 4, ql=[512] * 4, H=24, KVH=4, d=256, bs=16, dtype="bf16", seed=1006)


def prefix_flops(ctx, ql, H, d):
    """4 d flops (q.K and p.V) per visible (row, key) pair: row (j, h) sees ctx + j + 1 keys."""
    return sum(4 * d * H * (q * c + q * (q + 1) // 2) for c, q in zip(ctx, ql))


def measured_prefix_traffic():
    """HBM bytes per prefix-attention launch (scaled FETCH_SIZE + WRITE_SIZE)
    from the committed summary, or None when there is none or it was taken on
    different kernel sources."""
    from decode_attention_paged_v2_amd import rocprof_harness
    path = os.path.join(ROOT, "profiles", "prefix_attention.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    if data.get("source_hash") != rocprof_harness.source_hash() or "traffic_bytes" not in data:
        return None
    return round(float(data["traffic_bytes"]))


def prefix_bench(args, dev):
    """Paged prefix attention over a chunked prefill (the chunk's keys and
    values written into the cache first, outside the timed region)."""
    pav2.load()
    c = PREFIX_CASE
    pw = W.prefix_workload(c["ctx"], c["ql"], c["H"], c["KVH"], c["d"], c["bs"], dtype=c["dtype"], seed=c["seed"],
                           device=dev)
    pav2.reshape_and_cache(pw.key, pw.value, pw.key_cache, pw.value_cache, pw.slot_mapping)
    out = torch.empty_like(pw.query)
    max_seq = max(a + b for a, b in zip(c["ctx"], c["ql"]))
    stream = torch.cuda.current_stream(dev)
    fn = lambda: pav2.paged_prefix_attention(out, pw.query, pw.key_cache, pw.value_cache, pw.block_tables,
                                             pw.query_start_loc, pw.context_lens, max(c["ql"]), max_seq)
    mean, mn, wall = _time_launches(fn, args.steps, args.warmup, stream)
    flops = prefix_flops(c["ctx"], c["ql"], c["H"], c["d"])
    eb = 2 if c["dtype"] != "f32" else 4
    kv_bytes = sum((a + b) for a, b in zip(c["ctx"], c["ql"])) * c["KVH"] * 2 * c["d"] * eb
    tflops = flops / (mean * 1e-3) / 1e12
    result = {
        "metric": "paged prefix attention TFLOP/s (chunked prefill) and % of bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(mean, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": "4 seqs x (16384 cached + 512 new tokens), H=24, kv_h=4 (GQA 6), d=256, bf16, "
                               "block 16", "num_seqs": 4, "context": 16384, "chunk": 512},
        "ms_min": round(mn, 5), "wall_ms_per_launch": round(wall, 5),
        "kv_GBps_if_read_once": round(kv_bytes / (mean * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_prefix_traffic(),
                     "kernel": "phase1_kernel (prefix)", "algorithmic_flops_per_launch": flops},
        "library": pav2.lib_path(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefix_cpu_baseline(pw, c)
    return result


def prefix_cpu_baseline(pw, c, n_rows=12):
    """The oracle on the first n_rows chunk tokens of sequence 0 (one host thread)."""
    import oracle
    host = pw.to("cpu")
    n = n_rows
    t0 = time.perf_counter()
    oracle.prefix_attention(host.query[:n], host.key[:n], host.value[:n], host.key_cache, host.value_cache,
                            host.block_tables[:1], torch.tensor([0, n], dtype=torch.int32), host.context_lens[:1],
                            num_kv_heads=c["KVH"], block_size=c["bs"], scale=c["d"] ** -0.5,
                            q_dtype=oracle.BF16, kv_dtype=oracle.BF16)
    dt = time.perf_counter() - t0
    flops = prefix_flops([c["ctx"][0]], [n], c["H"], c["d"])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} chunk tokens of sequence 0 (all 24 heads), float64 C oracle, {dt:.2f} s wall",
            "seconds": round(dt, 3)}


def measured_cache_traffic(config):
    """HBM bytes per cache-write launch from the committed counter summary, or
    None when there is none or it was taken on different kernel sources."""
    from decode_attention_paged_v2_amd import rocprof_harness
    path = os.path.join(ROOT, "profiles", f"cache_write_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    if data.get("source_hash") != rocprof_harness.source_hash("cache_write") or "traffic_bytes" not in data:
        return None
    return round(float(data["traffic_bytes"]))


def copy_reference(dev, steps, warmup, nbytes=1 << 30):
    """A plain device-to-device copy of nbytes: reads nbytes, writes nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 5),
            "read_plus_write_GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_gqa", choices=list(W.SPECS))
    ap.add_argument("--entry", default="v2", choices=["v2", "v1", "auto"],
                    help="v2: both phases (the default); v1: the single-pass entry point; "
                         "auto: the planner's choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="extra per-step timings with a 1 GiB cache flush before each step")
    ap.add_argument("--mode", default="decode", choices=["decode", "copy", "cache_write", "prefix"],
                    help="copy: time a plain 1 GiB device copy (the reference kernel for "
                         "scaling HBM byte counters and for achievable bandwidth); cache_write: "
                         "time the KV-cache write of the workload's whole context (and of one "
                         "decode step's tokens); prefix: time paged prefix attention for a "
                         "chunked prefill")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; "
                          "--gpus above 1 is not supported"}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "copy":
        print(json.dumps(copy_reference(dev, args.steps, args.warmup)), flush=True)
        return
    if args.mode == "cache_write":
        print(json.dumps(cache_write_bench(args, dev)), flush=True)
        return
    if args.mode == "prefix":
        print(json.dumps(prefix_bench(args, dev)), flush=True)
        return
    pav2.load()
    spec = W.SPECS[args.config]
    t0 = time.time()
    wl = W.generate(spec, device=dev, poison=False)
    gen_s = time.time() - t0

    S, H, D, P = wl.num_seqs, wl.num_heads, wl.head_size, wl.max_num_partitions
    out = torch.empty_like(wl.query)
    es = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    ml = torch.empty_like(es)
    tmp = torch.empty((S, H, P, D), dtype=wl.q_dtype, device=dev)
    a = (wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads, wl.scale, wl.block_tables,
         wl.seq_lens, wl.block_size, wl.max_seq_len)
    kw = dict(alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale)
    stream = torch.cuda.current_stream(dev)
    plan = pav2.plan(S, H, wl.num_kv_heads, D, wl.block_size, P, pav2._binding._dtype_code(wl.query),
                     pav2._binding._dtype_code(wl.key_cache))
    entry = args.entry if args.entry != "auto" else ("v1" if plan["use_v1"] else "v2")

    def step(ev_a=None, ev_b=None, ev_c=None):
        if ev_a is not None:
            ev_a.record(stream)
        if entry == "v1":
            pav2.paged_attention_v1(out, *a, **kw)
        else:
            pav2.phase1(es, ml, tmp, *a, **kw)
        if ev_b is not None:
            ev_b.record(stream)
        if entry == "v2":
            pav2.phase2(out, es, ml, tmp, wl.seq_lens)
        if ev_c is not None:
            ev_c.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # phase 1's own duration comes from HIP events on every EVENT_EVERY-th step
    # of the timed region: an event recorded between the two kernels adds a
    # few microseconds of queue work to its step, so not every step carries one
    ev = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
          for i in range(0, args.steps, EVENT_EVERY)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i in ev:
            step(*ev[i])
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p1_ms = [e0.elapsed_time(e1) for e0, e1, _ in ev.values()]
    p2_ms = [e1.elapsed_time(e2) for _, e1, e2 in ev.values()]
    ms_per_step = wall * 1e3 / args.steps

    # cold-cache timings: flush L2 and the 256 MB MALL with a 1 GiB write first
    cold = []
    if args.flush_steps > 0:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.flush_steps):
            scratch.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del scratch

    kv = wl.kv_bytes()
    b1 = accounting.workload_bytes(wl)["phase1" if entry == "v2" else "v1"]
    traffic = measured_traffic(args.config, entry)
    p1_mean = float(np.mean(p1_ms))
    achieved = b1 / (p1_mean * 1e-3) / 1e9
    value = kv / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": "decode attention KV GB/s and % of HBM peak (Qwen-style 100K ctx, GQA 6)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[wl.q_dtype] + ("" if wl.kv_dtype == wl.q_dtype else "+fp8_e4m3_kv"),
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCR[args.config]}", "num_seqs": S,
                   "num_heads": H, "num_kv_heads": wl.num_kv_heads, "head_size": D,
                   "block_size": wl.block_size, "max_seq_len": wl.max_seq_len,
                   "max_num_partitions": P, "partition_size": 512},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_heads_per_s": round(wl.tokens_heads() / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv,
        "entry": entry,
        "phase1_ms_mean": round(p1_mean, 5),
        "phase1_event_steps": len(p1_ms),
        "phase1_ms_min": round(float(np.min(p1_ms)), 5),
        "phase2_ms_mean": round(float(np.mean(p2_ms)), 5) if entry == "v2" else None,
        "cold_cache_step_ms_median": round(float(np.median(cold)), 5) if cold else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "phase1_kernel" + (" (single pass)" if entry == "v1" else ""),
                     "algorithmic_bytes_per_launch": b1},
        "generate_s": round(gen_s, 2),
        "library": pav2.lib_path(),
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(wl, out.cpu())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
