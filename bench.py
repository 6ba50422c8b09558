#!/usr/bin/env python3
"""Benchmark PagedAttention V2 decode on one MI355X.

A step is one pass of the whole hot path over one batch: phase 1 (the
per-partition kernel) and phase 2 (the log-sum-exp combine), launched through
the C ABI on the current stream, on synthetic inputs already resident in HBM.

Timing: before every timed step a read sweep of 1 GiB with ordinary loads
evicts L2 and the 256 MB Infinity Cache (without leaving dirty lines behind);
a HIP event pair on the launch stream brackets phase 1 + phase 2 of the step.
`ms_per_step` is the median of those steps (min and mean reported too);
phase 1's own duration comes from a second pass of flushed steps with an
event between the two kernels.  A warm pass (back-to-back steps, host wall
clock) is reported as a secondary figure.

Default run: the long-context GQA decode the metric names (4 sequences x
100000 tokens, 24 query heads over 4 kv heads, head size 256, bf16, block
size 16) as the headline; a `configs` map with the same measurement for all
five workloads (step times, KV GB/s, % of 8 TB/s, and the error of sampled
(sequence, head) outputs against the float64 oracle); the block-sparse
decode of the long-context workload (attended bytes only); the chip's
achievable read bandwidth (a plain non-temporal read stream); and the CPU
oracle baseline.  `--config` selects another headline workload, `--single`
measures that workload alone, `--entry v1 | auto` times the single-pass entry
point or the planner's choice.

Prints ONE JSON line.  `value` is KV bytes read per second (decimal GB/s);
`roofline` reports phase 1's algorithmic bytes per launch over its mean
flushed duration against MI355X's 8 TB/s HBM peak.
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
FLUSH_BYTES = 1 << 30          # read sweep between timed steps (> L2 + Infinity Cache)
STREAM_BYTES = 4 << 30         # buffer of the achievable-bandwidth read stream
ORACLE_TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 2e-3}

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
    name = {"v2": "phase1_", "v1": "v1_", "blocksparse": "blocksparse_"}[entry] + config + ".json"
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
    if data.get("source_hash") != rocprof_harness.source_hash("prefix") or "traffic_bytes" not in data:
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
    # the key-range split's workspace, allocated once outside the timed region
    ws_bytes = pav2.prefix_workspace_bytes(pw.query, pw.key_cache, pw.value_cache, pw.context_lens, max(c["ql"]),
                                           max_seq)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    gqa = c["H"] // c["KVH"]
    num_work = len(c["ctx"]) * c["KVH"] * -(-max(c["ql"]) * gqa // 128)
    splits = ws_bytes // (num_work * 128 * (c["d"] + 2) * 4) if ws_bytes else 1
    fn = lambda: pav2.paged_prefix_attention(out, pw.query, pw.key_cache, pw.value_cache, pw.block_tables,
                                             pw.query_start_loc, pw.context_lens, max(c["ql"]), max_seq,
                                             workspace=ws)
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
        "timing": "mean of back-to-back launches (HIP events around each call)",
        "ms_min": round(mn, 5), "wall_ms_per_launch": round(wall, 5),
        "kv_GBps_if_read_once": round(kv_bytes / (mean * 1e-3) / 1e9, 1),
        "key_range_splits": int(splits), "workspace_bytes": int(ws_bytes),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_prefix_traffic(),
                     "kernel": "prefix_kernel (+ prefix_merge_kernel when split: the call's time)",
                     "algorithmic_flops_per_launch": flops},
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


class Timer:
    """Flushed step timing on one stream: a read sweep of FLUSH_BYTES with
    ordinary loads before each step (outside the events), a HIP event pair
    around the step, and optionally an event between its two kernels."""

    def __init__(self, dev):
        self.dev = dev
        self.stream = torch.cuda.current_stream(dev)
        self.buf = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device=dev)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def flush(self):
        pav2.read_stream(self.buf[:FLUSH_BYTES // 4], self.sink, nontemporal=False, stream=self.stream)

    def cold(self, first, second=None, steps=20, split=False):
        """Per-step event times (ms) of first() [+ second()] after a flush; with
        split, also the times of first() alone and second() alone."""
        st = self.stream
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in ev:
            self.flush()
            e[0].record(st)
            first()
            if split:
                e[1].record(st)
            if second is not None:
                second()
            e[2].record(st)
        torch.cuda.synchronize()
        whole = [e[0].elapsed_time(e[2]) for e in ev]
        if not split:
            return whole
        return whole, [e[0].elapsed_time(e[1]) for e in ev], [e[1].elapsed_time(e[2]) for e in ev]

    def warm(self, fn, steps):
        """Host wall-clock ms per step of back-to-back fn() calls."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def read_bandwidth(self, reps=10):
        """The achievable read rate: a non-temporal 16-byte-load stream over STREAM_BYTES."""
        fn = lambda: pav2.read_stream(self.buf, self.sink, nontemporal=True, stream=self.stream)
        for _ in range(3):
            fn()
        ms = self.cold(fn, steps=reps)
        best, med = float(np.min(ms)), float(np.median(ms))
        return {"bytes": STREAM_BYTES, "kernel": "read_stream_kernel (non-temporal 16-byte loads, 4 workgroups / CU)",
                "ms_median": round(med, 5), "GBps_median": round(STREAM_BYTES / (med * 1e-3) / 1e9, 1),
                "GBps_best": round(STREAM_BYTES / (best * 1e-3) / 1e9, 1),
                "pct_of_hbm_peak": round(100 * STREAM_BYTES / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}


def _stats(ms):
    return {"median": round(float(np.median(ms)), 5), "min": round(float(np.min(ms)), 5),
            "mean": round(float(np.mean(ms)), 5)}


def sample_pairs(wl, n=6, seed=0):
    """(sequence, head) pairs for the oracle check: the longest sequence's first
    and last head, an empty sequence if there is one, and random others."""
    rng = np.random.default_rng(seed)
    n = min(n, wl.num_seqs * wl.num_heads)
    lens = wl.seq_lens_host
    s_max = int(np.argmax(lens))
    pairs = [(s_max, 0), (s_max, wl.num_heads - 1)]
    empty = [s for s, L in enumerate(lens) if L == 0]
    if empty:
        pairs.append((empty[0], 0))
    while len(pairs) < n:
        p = (int(rng.integers(wl.num_seqs)), int(rng.integers(wl.num_heads)))
        if p not in pairs:
            pairs.append(p)
    return pairs


def oracle_error(wl, out_gpu, pairs, sparse=None):
    """Max |gpu - RNE(oracle)| over the pairs' outputs (float64 C oracle, threaded)."""
    import oracle
    host = wl.to("cpu")
    kw = dict(num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
              max_num_partitions=wl.max_num_partitions, q_dtype=oracle.dtype_code(wl.q_dtype),
              kv_dtype=oracle.dtype_code(wl.kv_dtype), alibi_slopes=host.alibi_slopes,
              k_scale=wl.k_scale, v_scale=wl.v_scale, pairs=pairs, threads=min(16, os.cpu_count() or 1))
    if sparse is not None:
        kw.update(tp_rank=sparse[0], blocksparse_local_blocks=sparse[1], blocksparse_vert_stride=sparse[2],
                  blocksparse_block_size=sparse[3], blocksparse_head_sliding_step=sparse[4])
    t0 = time.perf_counter()
    r = oracle.paged_attention_v2(host.query, host.key_cache, host.value_cache, host.block_tables,
                                  host.seq_lens, **kw)
    dt = time.perf_counter() - t0
    err = 0.0
    for s, h in pairs:
        ref = torch.from_numpy(r["out"][s, h]).to(wl.q_dtype).double()
        err = max(err, float((out_gpu[s, h].double() - ref).abs().max()))
    tol = 1e-2 if wl.kv_dtype == torch.float8_e4m3fn else ORACLE_TOL[wl.q_dtype]
    return {"pairs": len(pairs), "max_abs_err_vs_rounded_oracle": err, "tolerance": tol, "oracle_s": round(dt, 2)}


def measure_decode(name, dev, timer, steps, warmup, entry="v2", sparse=None, check=True):
    """Flushed and warm step times of one workload (V2 both phases, the single
    pass, or block-sparse V2), with sampled oracle errors."""
    spec = W.SPECS[name]
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
    kw = dict(alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale,
              kv_cache_dtype="fp8_e4m3" if wl.kv_dtype == torch.float8_e4m3fn else "auto")
    plan = pav2.plan(S, H, wl.num_kv_heads, D, wl.block_size, P, pav2._binding._dtype_code(wl.query),
                     pav2._binding._dtype_code(wl.key_cache))
    if entry == "auto":
        entry = "v1" if plan["use_v1"] else "v2"
    if sparse is not None:
        sk = dict(tp_rank=sparse[0], blocksparse_local_blocks=sparse[1], blocksparse_vert_stride=sparse[2],
                  blocksparse_block_size=sparse[3], blocksparse_head_sliding_step=sparse[4])
        first = lambda: pav2.phase1_blocksparse(es, ml, tmp, *a, **kw, **sk)
        second = lambda: pav2.phase2(out, es, ml, tmp, wl.seq_lens)
        acct = accounting.blocksparse_workload_bytes(wl, sparse)
        kv, b1 = acct["kv"], acct["phase1"]
    elif entry == "v1":
        first, second = (lambda: pav2.paged_attention_v1(out, *a, **kw)), None
        acct = accounting.workload_bytes(wl)
        kv, b1 = acct["kv"], acct["v1"]
    else:
        first = lambda: pav2.phase1(es, ml, tmp, *a, **kw)
        second = lambda: pav2.phase2(out, es, ml, tmp, wl.seq_lens)
        acct = accounting.workload_bytes(wl)
        kv, b1 = acct["kv"], acct["phase1"]
    step = (lambda: (first(), second())) if second is not None else first
    for _ in range(warmup):
        timer.flush()
        step()
    whole = timer.cold(first, second, steps)
    res = {"workload": f"{name}: {DESCR[name]}", "entry": "blocksparse" if sparse is not None else entry,
           "planner_entry": "v1" if plan["use_v1"] else "v2", "generate_s": round(gen_s, 2),
           "kv_bytes_per_step": kv, "step_ms": _stats(whole)}
    med = float(np.median(whole))
    res["kv_GBps"] = round(kv / (med * 1e-3) / 1e9, 2)
    res["pct_of_hbm_peak"] = round(100.0 * kv / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
    res["tokens_heads_per_s"] = round(wl.tokens_heads() / (med * 1e-3), 1)
    if second is not None:
        _, p1, p2 = timer.cold(first, second, steps, split=True)
        res["phase1_ms"] = _stats(p1)
        res["phase2_ms"] = _stats(p2)
    elif b1 is not None:
        res["phase1_ms"] = _stats(whole)     # one launch: the single pass is the step
    if b1 is not None:
        res["phase1_algorithmic_bytes"] = b1
        res["phase1_GBps"] = round(b1 / (res["phase1_ms"]["mean"] * 1e-3) / 1e9, 2)
    res["warm_ms_per_step"] = round(timer.warm(step, steps), 5)
    if check:
        torch.cuda.synchronize()
        res["oracle_check"] = oracle_error(wl, out.cpu(), sample_pairs(wl), sparse)
    print(f"[bench] {name}{' block-sparse' if sparse is not None else ''} ({res['entry']}): step median "
          f"{res['step_ms']['median']:.4f} ms, {res['pct_of_hbm_peak']:.1f} % of 8 TB/s", file=sys.stderr, flush=True)
    return res, wl, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_gqa", choices=list(W.SPECS))
    ap.add_argument("--entry", default="auto", choices=["v2", "v1", "auto"],
                    help="auto (the default): the library's V1 / V2 dispatch (forward_decode's plan); "
                         "v2: both phases; v1: the single-pass entry point")
    ap.add_argument("--single", action="store_true",
                    help="measure the --config workload alone (no configs map, block-sparse line or "
                         "read-stream figure, no oracle check)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="decode", choices=["decode", "blocksparse", "copy", "cache_write", "prefix"],
                    help="blocksparse: the block-sparse decode of the workload; copy: time a plain 1 GiB "
                         "device copy (the reference kernel for scaling HBM byte counters); cache_write: "
                         "time the KV-cache write of the workload's whole context (and of one decode step's "
                         "tokens); prefix: time paged prefix attention for a chunked prefill")
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
    timer = Timer(dev)
    if args.mode == "blocksparse":
        print(json.dumps(blocksparse_line(args, dev, timer)), flush=True)
        return

    head, wl, out = measure_decode(args.config, dev, timer, args.steps, args.warmup, args.entry,
                                   check=not args.single)
    entry = head["entry"]
    med = head["step_ms"]["median"]
    traffic = measured_traffic(args.config, entry)
    b1 = head["phase1_algorithmic_bytes"]
    achieved = head["phase1_GBps"]
    result = {
        "metric": "decode attention KV GB/s and % of HBM peak (Qwen-style 100K ctx, GQA 6)",
        "value": head["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[wl.q_dtype] + ("" if wl.kv_dtype == wl.q_dtype else "+fp8_e4m3_kv"),
        "data": "synthetic",
        "config": {"workload": head["workload"], "num_seqs": wl.num_seqs,
                   "num_heads": wl.num_heads, "num_kv_heads": wl.num_kv_heads, "head_size": wl.head_size,
                   "block_size": wl.block_size, "max_seq_len": wl.max_seq_len,
                   "max_num_partitions": wl.max_num_partitions, "partition_size": 512},
        "timing": "median of flushed steps (1 GiB read sweep before each, HIP events around phase 1 + phase 2)",
        "pct_of_hbm_peak": head["pct_of_hbm_peak"],
        "tokens_heads_per_s": head["tokens_heads_per_s"],
        "kv_bytes_per_step": head["kv_bytes_per_step"],
        "entry": entry,
        "step_ms": head["step_ms"],
        "phase1_ms": head.get("phase1_ms"),
        "phase2_ms": head.get("phase2_ms"),
        "warm_ms_per_step": head["warm_ms_per_step"],
        "warm_kv_GBps": round(head["kv_bytes_per_step"] / (head["warm_ms_per_step"] * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "phase1_kernel" + (" (single pass)" if entry == "v1" else ""),
                     "algorithmic_bytes_per_launch": b1},
        "generate_s": head["generate_s"],
        "library": pav2.lib_path(),
    }
    if "oracle_check" in head:
        result["oracle_check"] = head["oracle_check"]
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(wl, out.cpu())
        result["cpu_baseline"]["single_thread_tiny"] = single_thread_tiny()
    del wl, out
    torch.cuda.empty_cache()
    if not args.single:
        result["achievable_read"] = timer.read_bandwidth()
        configs = {}
        for name in W.SPECS:
            if name == args.config:
                configs[name] = {k: head[k] for k in ("step_ms", "kv_GBps", "pct_of_hbm_peak", "phase1_ms",
                                                      "phase2_ms", "warm_ms_per_step", "planner_entry",
                                                      "oracle_check") if k in head}
                continue
            r, _, _ = measure_decode(name, dev, timer, args.steps, args.warmup, args.entry)
            configs[name] = {k: r[k] for k in ("step_ms", "kv_GBps", "pct_of_hbm_peak", "phase1_ms", "phase2_ms",
                                               "warm_ms_per_step", "planner_entry", "oracle_check") if k in r}
            torch.cuda.empty_cache()
        result["configs"] = configs
        bs, _, _ = measure_decode("long_gqa", dev, timer, args.steps, args.warmup, sparse=BLOCKSPARSE_PATTERN)
        result["blocksparse"] = {"pattern": dict(zip(("tp_rank", "local_blocks", "vert_stride", "block_size",
                                                       "head_sliding_step"), BLOCKSPARSE_PATTERN)),
                                 **{k: bs[k] for k in ("workload", "kv_bytes_per_step", "step_ms", "kv_GBps",
                                                       "pct_of_hbm_peak", "phase1_ms", "phase1_GBps", "phase2_ms",
                                                       "warm_ms_per_step", "oracle_check")}}
    print(json.dumps(result), flush=True)


def blocksparse_line(args, dev, timer):
    """Block-sparse V2 on the chosen workload with the benchmark pattern: KV
    bytes are the attended ones (per kv-head group, the tokens some head attends)."""
    r, wl, _ = measure_decode(args.config, dev, timer, args.steps, args.warmup, sparse=BLOCKSPARSE_PATTERN,
                              check=not args.single)
    med = r["step_ms"]["median"]
    return {
        "metric": "block-sparse decode attention: attended KV GB/s and % of HBM peak",
        "value": r["kv_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": med, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[wl.q_dtype], "data": "synthetic",
        "config": {"workload": r["workload"] + " with 64-token sparse blocks: a 16-block local window and every "
                                               "8th block, the same stripes for every head",
                   "pattern": dict(zip(("tp_rank", "local_blocks", "vert_stride", "block_size",
                                        "head_sliding_step"), BLOCKSPARSE_PATTERN))},
        "pct_of_hbm_peak": r["pct_of_hbm_peak"], "kv_bytes_per_step": r["kv_bytes_per_step"],
        "dense_kv_bytes": wl.kv_bytes(), "step_ms": r["step_ms"], "warm_ms_per_step": r["warm_ms_per_step"],
        "phase1_ms": r["phase1_ms"], "phase2_ms": r["phase2_ms"],
        "roofline": {"bound": "hbm", "achieved": r["phase1_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(r["phase1_GBps"] / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.config, "blocksparse"),
                     "kernel": "phase1_kernel (block-sparse)",
                     "algorithmic_bytes_per_launch": r["phase1_algorithmic_bytes"]},
        **({"oracle_check": r["oracle_check"]} if "oracle_check" in r else {}),
        "library": pav2.lib_path(),
    }


def single_thread_tiny():
    """The oracle on the whole tiny workload (1 x 1000 tokens, 4 heads) on one host thread."""
    import oracle
    wl = W.generate(W.SPECS["tiny"], poison=False)
    t0 = time.perf_counter()
    oracle.paged_attention_v2(wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.seq_lens,
                              num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
                              max_num_partitions=wl.max_num_partitions, q_dtype=oracle.F32, kv_dtype=oracle.F32,
                              threads=1)
    dt = time.perf_counter() - t0
    return {"workload": "tiny: " + DESCR["tiny"], "cores": 1, "seconds": round(dt, 4),
            "GBps": round(wl.kv_bytes() / dt / 1e9, 4), "tokens_heads_per_s": round(wl.tokens_heads() / dt, 1)}


if __name__ == "__main__":
    main()
