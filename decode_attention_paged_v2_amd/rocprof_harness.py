"""rocprofv3 harness: per-kernel durations and HBM traffic of the decode path.

    python -m decode_attention_paged_v2_amd.rocprof_harness --config long_gqa \
        --out gpurun_out/prof [--pmc] [--sq] [--entry v1]

Runs `bench.py` (a few steps, no CPU baseline) under

* `rocprofv3 --kernel-trace --stats` -> average / min / max duration of the
  phase-1 and phase-2 kernels;
* with `--pmc`, two counter passes (`FETCH_SIZE`, then `WRITE_SIZE`, KiB per
  dispatch) over the same command and over `bench.py --mode copy` (a plain
  1 GiB copy).  Each counter is scaled by the ratio of the copy's known bytes
  to what the counter reports for it, giving HBM bytes per phase-1 launch;
* with `--sq`, two passes of SQ instruction counters over phase 1, reported
  per (work item, wavefront);
* with `--entry v1`, the same over the single-pass entry point (one launch
  per step, priced with that entry point's algorithmic bytes).

Writes `<out>/<kernel>_<config>.md` (`phase1_`, or `v1_` for the single pass) (a short summary with the commands) and
`<out>/<kernel>_<config>.json` (the numbers, plus a hash of the kernel sources
so that bench.py can tell whether the counters still describe the current
kernel).  rocprofv3 runs as a child process from /tmp with TMPDIR=/tmp; this
module never touches the GPU itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BENCH = os.path.join(ROOT, "bench.py")
# What a summary's counters depend on: the kernels, and the launch plan in the
# C ABI (schedule choice, grid sizes, LDS bytes, scale folding).
_PLAN = [os.path.join(HERE, "csrc", "api.hip"), os.path.join(ROOT, "include", "pav2.h")]
KERNEL_SOURCES = {
    "decode": sorted(glob.glob(os.path.join(HERE, "csrc", "phase1*"))) +
              [os.path.join(HERE, "csrc", f) for f in ("phase2.hip", "pav2_internal.h")] + _PLAN,
    "prefix": [os.path.join(HERE, "csrc", f) for f in ("prefix.hip", "prefix.h", "pav2_internal.h")] + _PLAN,
    "cache_write": [os.path.join(HERE, "csrc", f) for f in ("cache.hip", "cache.h", "pav2_internal.h")] + _PLAN,
}


def source_hash(mode: str = "decode") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[mode]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run(cmd, log, timeout):
    env = dict(os.environ, TMPDIR="/tmp")
    print("[harness] " + " ".join(cmd), flush=True)
    with open(log, "w") as fh:
        p = subprocess.Popen(cmd, stdout=fh, stderr=subprocess.STDOUT, cwd="/tmp", env=env,
                             start_new_session=True)
        try:
            rc = p.wait(timeout=timeout)
        except subprocess.TimeoutExpired:
            os.killpg(p.pid, 9)
            p.wait()
            raise RuntimeError(f"timed out: {' '.join(cmd)}")
    if rc != 0:
        with open(log) as fh:
            tail = fh.read()[-2000:]
        raise RuntimeError(f"rc={rc}: {' '.join(cmd)}\n{tail}")


def _csv(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise RuntimeError(f"no file matches {pattern}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _kind(name: str) -> str:
    if "prefix_merge_kernel" in name:
        return "prefix_merge"
    if "prefix_kernel" in name:
        return "prefix"
    if "phase1_kernel" in name:
        return "phase1"
    if "phase2_kernel" in name:
        return "phase2"
    if "cache_write_kernel" in name:
        return "cache_write"
    return "other"


def _bench_args(config: str, mode: str, steps: int, warmup: int, entry: str = "v2") -> list:
    args = [sys.executable, BENCH, "--config", config, "--steps", str(steps), "--warmup", str(warmup),
            "--no-cpu-baseline"]
    if mode in ("cache_write", "prefix"):
        return args + ["--mode", mode]
    # the benchmark's own flushed steps (a read sweep before each), one workload
    args = args + ["--single"]
    if mode == "blocksparse":
        return args + ["--mode", "blocksparse"]
    return args + ["--entry", "v1" if entry == "v1" else "v2"]   # (the bench's default is the planner's choice)


def _tag(mode: str, config: str, entry: str) -> str:
    if mode == "prefix":   # one fixed case, no --config
        return mode
    return f"{mode}_{config}" if entry == "v2" else f"{mode}_v1_{config}"


def kernel_trace(config: str, out: str, steps: int = 10, mode: str = "decode", entry: str = "v2") -> dict:
    d = os.path.join(out, "trace_" + _tag(mode, config, entry))
    shutil.rmtree(d, ignore_errors=True)
    # prefix attention: the benchmark's own 5 warm-up and 50 timed launches, so
    # that the trace's average covers the calls the benchmark's mean covers
    bench = _bench_args(config, mode, steps, 5 if mode == "prefix" else 2, entry)
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "-d", d, "-o", "run", "--output-format", "csv",
           "--"] + bench
    _run(cmd, d + ".log", 300)
    rel = os.path.relpath(d, ROOT)
    res = {"command": " ".join(["rocprofv3", "--kernel-trace", "--stats", "-d", rel, "-o", "run",
                                "--output-format", "csv", "--", "python3", "bench.py"] + bench[2:])}
    if mode == "cache_write":
        # the bench times the whole-context write and a decode step's write with
        # the same kernel: keep the dispatches of the largest grid (the former)
        rows = [r for r in _csv(os.path.join(d, "**", "run_kernel_trace.csv"))
                if _kind(r["Kernel_Name"]) == "cache_write"]
        size = lambda r: int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"])
        top = max(size(r) for r in rows)
        us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if size(r) == top]
        res["cache_write"] = {"name": rows[0]["Kernel_Name"], "calls": len(us), "avg_us": sum(us) / len(us),
                              "min_us": min(us), "max_us": max(us), "grid": top}
        return res
    for r in _csv(os.path.join(d, "**", "run_kernel_stats.csv")):
        k = _kind(r["Name"])
        if k == "other":
            continue
        res[k] = {"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                  "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    # per-dispatch durations: the median, which a clock transient over the
    # first back-to-back calls (seen on long compute-bound launches) does not move
    per = {}
    for r in _csv(os.path.join(d, "**", "run_kernel_trace.csv")):
        k = _kind(r["Kernel_Name"])
        if k in res:
            per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k, us in per.items():
        us.sort()
        res[k]["median_us"] = (us[(len(us) - 1) // 2] + us[len(us) // 2]) / 2
    return res


def pmc(config: str, out: str, mode: str = "decode", entry: str = "v2") -> dict:
    """FETCH_SIZE and WRITE_SIZE per launch of the profiled kernels, scaled by the copy reference."""
    res = {}
    # the single-pass entry point launches the phase-1 kernel template only
    kinds = {"cache_write": ("cache_write",), "prefix": ("prefix", "prefix_merge")}.get(
        mode, ("phase1",) if entry == "v1" else ("phase1", "phase2"))
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        for what in (config, "copy"):
            d = os.path.join(out, f"pmc_{counter}_" + ("copy" if what == "copy" else _tag(mode, what, entry)))
            shutil.rmtree(d, ignore_errors=True)
            if what == "copy":
                bench = [sys.executable, BENCH, "--mode", "copy", "--steps", "3", "--warmup", "1"]
            else:
                bench = _bench_args(what, mode, 3, 1, entry)
            cmd = ["rocprofv3", "--pmc", counter, "-d", d, "-o", "run", "--output-format", "csv",
                   "--"] + bench
            _run(cmd, d + ".log", 120)
            rows = _csv(os.path.join(d, "**", "run_counter_collection.csv"))
            if what == "copy":
                vals = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
                # the reference copy moves 1 GiB each way
                res[f"{counter}_copy_kib"] = sum(vals) / len(vals)
                res[f"{counter}_scale"] = (1 << 30) / 1024.0 / res[f"{counter}_copy_kib"]
            else:
                for k in kinds:
                    # dispatches of the largest grid (the cache write also times a decode step)
                    mine = [r for r in rows if _kind(r["Kernel_Name"]) == k]
                    if not mine:   # (an unsplit prefix call launches no merge)
                        res[f"{counter}_{k}_kib"] = 0.0
                        continue
                    top = max(int(r["Grid_Size"]) for r in mine)
                    vals = [float(r["Counter_Value"]) for r in mine if int(r["Grid_Size"]) == top]
                    res[f"{counter}_{k}_kib"] = sum(vals) / len(vals)
    for k in kinds:
        res[f"{k}_fetch_bytes"] = res[f"FETCH_SIZE_{k}_kib"] * 1024 * res["FETCH_SIZE_scale"]
        res[f"{k}_write_bytes"] = res[f"WRITE_SIZE_{k}_kib"] * 1024 * res["WRITE_SIZE_scale"]
    return res


SQ_PASSES = [
    ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "SQ_INSTS_SALU"],
    ["SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SMEM", "SQ_INSTS_BRANCH"],
]


def sq(config: str, out: str) -> dict:
    """Instruction mix of phase 1: kernel-wide SQ instruction counts, two passes."""
    vals = {}
    for i, counters in enumerate(SQ_PASSES):
        d = os.path.join(out, f"sq{i}_{config}")
        shutil.rmtree(d, ignore_errors=True)
        bench = [sys.executable, BENCH, "--config", config, "--steps", "3", "--warmup", "1",
                 "--no-cpu-baseline", "--single", "--entry", "v2"]
        cmd = ["rocprofv3", "--pmc", *counters, "-d", d, "-o", "run", "--output-format", "csv", "--"] + bench
        _run(cmd, os.path.join(out, f"sq{i}_{config}.log"), 120)
        per = {}
        for r in _csv(os.path.join(d, "**", "run_counter_collection.csv")):
            if _kind(r["Kernel_Name"]) != "phase1":
                continue
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for k, v in per.items():
            vals[k] = sum(v) / len(v)
        vals.setdefault("commands", []).append(
            f"rocprofv3 --pmc {' '.join(counters)} -d gpurun_out/prof/sq{i}_{config} -o run "
            f"--output-format csv -- python3 bench.py {' '.join(bench[2:])}")
    return vals


def phase1_waves(config: str) -> int:
    """Wavefronts per phase-1 workgroup, from the library's host-side launch plan."""
    from . import _binding as B, workloads
    sp = workloads.SPECS[config]
    code = {"f32": B.F32, "f16": B.F16, "bf16": B.BF16, "fp8_e4m3": B.FP8_E4M3}
    pl = B.plan(1, sp.num_heads, sp.num_kv_heads, sp.head_size, sp.block_size, 1,
                code[sp.q_dtype], code[sp.kv_dtype])
    return pl["phase1_threads"] // 64


def algorithmic_bytes(config: str) -> dict:
    """Phase-1 / phase-2 algorithmic bytes of the workload (host-side, no GPU)."""
    from . import accounting, workloads
    return accounting.spec_bytes(workloads.SPECS[config])


def write_summary(config: str, out: str, trace: dict, counters: dict | None, sqv: dict | None = None,
                  entry: str = "v2") -> str:
    alg = dict(algorithmic_bytes(config))
    if entry == "blocksparse":
        # the attended K/V only (the benchmark's pattern)
        from . import accounting, workloads
        import bench
        alg = dict(accounting.blocksparse_spec_bytes(workloads.SPECS[config], bench.BLOCKSPARSE_PATTERN))
    if entry == "v1":
        # the single pass reads what phase 1 reads and writes the final rows only
        alg["phase1"] = alg["v1"]
        alg["phase1_write"] = alg["v1"] - alg["phase1_read"]
    p1 = trace["phase1"]
    name = {"v2": "phase1_", "v1": "v1_", "blocksparse": "blocksparse_"}[entry] + config
    title = {"v2": "Phase 1 / phase 2", "v1": "Single-pass (V1)", "blocksparse": "Block-sparse phase 1 / phase 2"}[entry]
    label = {"v2": "Phase-1", "v1": "Single-pass", "blocksparse": "Block-sparse phase-1"}[entry]
    lines = [f"# {title} profile: {config}", "",
             f"Kernel sources hash: `{source_hash()}`", "",
             "Kernel trace command (from the repository root):", "",
             "    python -m decode_attention_paged_v2_amd.rocprof_harness --config "
             f"{config}{' --entry v1' if entry == 'v1' else ''}"
             f"{' --mode blocksparse' if entry == 'blocksparse' else ''} --out gpurun_out/prof"
             f"{' --pmc' if counters else ''}{' --sq' if sqv else ''}", "",
             "which runs:", "", "    " + trace["command"], "",
             "| kernel | calls | average (µs) | min (µs) | max (µs) |", "|---|---|---|---|---|"]
    for k in ("phase1", "phase2"):
        t = trace.get(k)
        if t:
            lines.append(f"| `{t['name'][:90]}` | {t['calls']} | {t['avg_us']:.2f} | {t['min_us']:.2f} | "
                         f"{t['max_us']:.2f} |")
    gbps = alg["phase1"] / (p1["avg_us"] * 1e-6) / 1e9
    lines += ["", f"{label} algorithmic bytes per launch: {alg['phase1']:,} "
                  f"(K/V {alg['kv']:,}); at the average duration that is {gbps:.1f} GB/s = "
                  f"{100 * gbps / 8000:.1f} % of 8 TB/s."]
    data = {"config": config, "entry": entry, "source_hash": source_hash(), "trace": trace, "algorithmic": alg,
            "phase1_achieved_GBps": gbps, "taken": time.strftime("%Y-%m-%d %H:%M:%S")}
    if counters:
        f1, w1 = counters["phase1_fetch_bytes"], counters["phase1_write_bytes"]
        data["counters"] = counters
        data["phase1_traffic_bytes"] = f1 + w1
        lines += ["", "HBM counters (`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, each over "
                      "the same bench command and over `bench.py --mode copy`, a 1 GiB copy):", "",
                  "| quantity | value |", "|---|---|",
                  f"| FETCH_SIZE of the 1 GiB copy (KiB) | {counters['FETCH_SIZE_copy_kib']:.1f} |",
                  f"| WRITE_SIZE of the 1 GiB copy (KiB) | {counters['WRITE_SIZE_copy_kib']:.1f} |",
                  f"| scale factors (known / counted) | fetch {counters['FETCH_SIZE_scale']:.4f}, "
                  f"write {counters['WRITE_SIZE_scale']:.4f} |",
                  f"| {label} FETCH_SIZE per launch (KiB, raw) | {counters['FETCH_SIZE_phase1_kib']:.1f} |",
                  f"| {label} WRITE_SIZE per launch (KiB, raw) | {counters['WRITE_SIZE_phase1_kib']:.1f} |",
                  f"| {label} HBM read bytes (scaled) | {f1:,.0f} |",
                  f"| {label} HBM write bytes (scaled) | {w1:,.0f} |",
                  f"| algorithmic reads / writes | {alg['phase1_read']:,} / {alg['phase1_write']:,} |",
                  f"| measured / algorithmic | reads {f1 / alg['phase1_read']:.4f}, "
                  f"writes {w1 / alg['phase1_write']:.4f} |"]
    if sqv:
        data["sq"] = sqv
        # every wavefront of a work item runs the same unrolled unit loop, so
        # counts per (item, wavefront) are the per-item instruction budget
        waves = phase1_waves(config)
        per = alg["phase1_items"] * waves
        lines += ["", f"Instruction mix of phase 1 (rocprofv3 `--pmc` SQ counters, kernel-wide totals "
                  f"divided by {alg['phase1_items']:,} work items x {waves} wavefronts):", ""]
        lines += ["    " + c for c in sqv["commands"]]
        lines += ["", "| counter | per (item, wavefront) |", "|---|---|"]
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA",
                  "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_SMEM", "SQ_INSTS_BRANCH"):
            if k in sqv:
                lines.append(f"| {k} | {sqv[k] / per:.1f} |")
    with open(os.path.join(out, name + ".md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(os.path.join(out, name + ".json"), "w") as fh:
        json.dump(data, fh, indent=1)
    return os.path.join(out, name + ".md")


def write_cache_summary(config: str, out: str, trace: dict, counters: dict | None) -> str:
    from . import workloads
    import torch
    sp = workloads.SPECS[config]
    gl = torch.Generator()
    gl.manual_seed(sp.seed)
    tokens = sum(int(v) for v in sp.lens(gl))
    eb = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
    rd = tokens * sp.num_kv_heads * sp.head_size * 2 * eb[sp.q_dtype]   # key and value read
    alg = rd + tokens * sp.num_kv_heads * sp.head_size * 2 * eb[sp.kv_dtype]
    t = trace["cache_write"]
    gbps = alg / (t["avg_us"] * 1e-6) / 1e9
    name = "cache_write_" + config
    lines = [f"# KV-cache write profile: {config} (whole context in one launch)", "",
             f"Kernel sources hash: `{source_hash('cache_write')}`", "",
             "Command (from the repository root):", "",
             "    python -m decode_attention_paged_v2_amd.rocprof_harness --mode cache_write --config "
             f"{config} --out gpurun_out/prof{' --pmc' if counters else ''}", "",
             "which runs:", "", "    " + trace["command"], "",
             "Dispatches of the largest grid (the whole-context write; the bench also times a decode "
             "step's write with the same kernel), from the kernel trace:", "",
             "| kernel | grid | calls | average (µs) | min (µs) | max (µs) |", "|---|---|---|---|---|---|",
             f"| `{t['name'][:90]}` | {t['grid']} | {t['calls']} | {t['avg_us']:.2f} | {t['min_us']:.2f} | "
             f"{t['max_us']:.2f} |", "",
             f"Algorithmic bytes per launch (input read + cache written): {alg:,}; at the average "
             f"duration that is {gbps:.1f} GB/s = {100 * gbps / 8000:.1f} % of 8 TB/s."]
    data = {"config": config, "source_hash": source_hash("cache_write"), "trace": trace,
            "algorithmic_bytes": alg, "achieved_GBps": gbps, "taken": time.strftime("%Y-%m-%d %H:%M:%S")}
    if counters:
        f1, w1 = counters["cache_write_fetch_bytes"], counters["cache_write_write_bytes"]
        data["counters"] = counters
        data["traffic_bytes"] = f1 + w1
        lines += ["", "HBM counters (`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, each over the "
                      "same bench command and over `bench.py --mode copy`, a 1 GiB copy):", "",
                  "| quantity | value |", "|---|---|",
                  f"| scale factors (known / counted) | fetch {counters['FETCH_SIZE_scale']:.4f}, "
                  f"write {counters['WRITE_SIZE_scale']:.4f} |",
                  f"| HBM read bytes per launch (scaled) | {f1:,.0f} |",
                  f"| HBM write bytes per launch (scaled) | {w1:,.0f} |",
                  f"| algorithmic reads / writes | {rd:,} / {alg - rd:,} |",
                  f"| measured / algorithmic | reads {f1 / rd:.4f}, writes {w1 / (alg - rd):.4f} |"]
    with open(os.path.join(out, name + ".md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(os.path.join(out, name + ".json"), "w") as fh:
        json.dump(data, fh, indent=1)
    return os.path.join(out, name + ".md")


def _bench_json(log: str) -> dict:
    """The bench's JSON line from a profiled run's log (the last line that parses); {} without one."""
    if not os.path.exists(log):
        return {}
    with open(log) as fh:
        for line in reversed(fh.read().splitlines()):
            if line.startswith("{"):
                try:
                    return json.loads(line)
                except ValueError:
                    continue
    return {}


def write_prefix_summary(out: str, trace: dict, counters: dict | None = None) -> str:
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_for_counts", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    c = bench.PREFIX_CASE
    flops = bench.prefix_flops(c["ctx"], c["ql"], c["H"], c["d"])
    t, tm = trace["prefix"], trace.get("prefix_merge")
    line = _bench_json(os.path.join(out, "trace_prefix.log"))
    splits, ws = line.get("key_range_splits", 1), line.get("workspace_bytes", 0)
    call_us = t["avg_us"] + (tm["avg_us"] if tm else 0.0)
    tf = flops / (t["avg_us"] * 1e-6) / 1e12
    tf_call = flops / (call_us * 1e-6) / 1e12
    med = lambda k: k.get("median_us", k["avg_us"])
    call_med = med(t) + (med(tm) if tm else 0.0)
    tf_med = flops / (med(t) * 1e-6) / 1e12
    tf_call_med = flops / (call_med * 1e-6) / 1e12
    name = "prefix_attention"
    lines = ["# Paged prefix attention profile: 4 seqs x (16384 cached + 512 new tokens), H=24, kv_h=4, d=256, bf16",
             "", f"Kernel sources hash: `{source_hash('prefix')}`", "",
             "Command (from the repository root):", "",
             "    python -m decode_attention_paged_v2_amd.rocprof_harness --mode prefix --out gpurun_out/prof"
             + (" --pmc" if counters else ""), "",
             "which runs:", "", "    " + trace["command"], "",
             f"Key ranges per row block: {splits} (workspace {ws:,} bytes); the call is the attention kernel "
             "and, when split, the merge kernel.", "",
             "| kernel | calls | average (µs) | median (µs) | min (µs) | max (µs) |", "|---|---|---|---|---|---|"]
    for k in (t, tm):
        if k:
            lines.append(f"| `{k['name'][:90]}` | {k['calls']} | {k['avg_us']:.2f} | {med(k):.2f} | "
                         f"{k['min_us']:.2f} | {k['max_us']:.2f} |")
    lines += ["", f"Algorithmic flops per call (4 d per visible (row, key) pair): {flops:,}.  At the attention "
                  f"kernel's average duration: {tf:.1f} TFLOP/s = {100 * tf / 2500:.2f} % of the 2.5 PFLOP/s bf16 "
                  f"MFMA peak; over the whole call ({call_us:.1f} µs): {tf_call:.1f} TFLOP/s = "
                  f"{100 * tf_call / 2500:.2f} %.",
              "", f"At the median durations (back-to-back calls first run slower for a few calls, then settle): "
                  f"attention kernel {tf_med:.1f} TFLOP/s = {100 * tf_med / 2500:.2f} %; whole call "
                  f"({call_med:.1f} µs) {tf_call_med:.1f} TFLOP/s = {100 * tf_call_med / 2500:.2f} %."]
    data = {"source_hash": source_hash("prefix"), "trace": trace, "algorithmic_flops": flops,
            "achieved_TFLOPs": tf, "achieved_TFLOPs_call": tf_call, "achieved_TFLOPs_median": tf_med,
            "achieved_TFLOPs_call_median": tf_call_med, "key_range_splits": splits,
            "workspace_bytes": ws, "taken": time.strftime("%Y-%m-%d %H:%M:%S")}
    if counters:
        # unique bytes: every (cached + new) token's K and V once, the queries,
        # the block-table rows and per-sequence metadata; writes: the output
        # rows, or the float32 partials when split (read back by the merge)
        eb = 4 if c["dtype"] == "f32" else 2
        rows = sum(c["ql"]) * c["H"] * c["d"] * eb
        tokens = sum(a + b for a, b in zip(c["ctx"], c["ql"]))
        blocks = sum(-(-(a + b) // c["bs"]) for a, b in zip(c["ctx"], c["ql"]))
        alg_r = tokens * c["KVH"] * 2 * c["d"] * eb + rows + 4 * blocks + 3 * 4 * len(c["ql"])
        alg_w = ws if splits > 1 else rows
        f, w = counters["prefix_fetch_bytes"], counters["prefix_write_bytes"]
        fm, wm = counters["prefix_merge_fetch_bytes"], counters["prefix_merge_write_bytes"]
        data["counters"] = counters
        data["traffic_bytes"] = f + w
        data["merge_traffic_bytes"] = fm + wm
        data["unique_read_bytes"], data["unique_write_bytes"] = alg_r, alg_w
        lines += ["", "HBM counters (`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, over the same bench "
                      "command and over `bench.py --mode copy`, a 1 GiB copy):", "",
                  "| quantity | value |", "|---|---|",
                  f"| scale factors (known / counted) | fetch {counters['FETCH_SIZE_scale']:.4f}, "
                  f"write {counters['WRITE_SIZE_scale']:.4f} |",
                  f"| attention kernel: FETCH_SIZE / WRITE_SIZE per launch (KiB, raw) | "
                  f"{counters['FETCH_SIZE_prefix_kib']:.1f} / {counters['WRITE_SIZE_prefix_kib']:.1f} |",
                  f"| attention kernel: HBM read / write bytes (scaled) | {f:,.0f} / {w:,.0f} |",
                  f"| unique reads (K/V of every token once, queries, tables) / writes (output, or the "
                  f"partials when split) | {alg_r:,} / {alg_w:,} |",
                  f"| attention kernel: measured / unique | reads {f / alg_r:.4f}, writes {w / alg_w:.4f} |"]
        if tm:
            lines.append(f"| merge kernel: HBM read / write bytes (scaled) | {fm:,.0f} / {wm:,.0f} |")
    with open(os.path.join(out, name + ".md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(os.path.join(out, name + ".json"), "w") as fh:
        json.dump(data, fh, indent=1)
    return os.path.join(out, name + ".md")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="long_gqa")
    ap.add_argument("--mode", default="decode", choices=["decode", "blocksparse", "cache_write", "prefix"])
    ap.add_argument("--out", default="gpurun_out/prof")
    ap.add_argument("--pmc", action="store_true", help="HBM FETCH_SIZE / WRITE_SIZE passes")
    ap.add_argument("--sq", action="store_true", help="instruction-mix / utilisation passes")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 10; prefix mode 50)")
    ap.add_argument("--entry", default="v2", choices=["v2", "v1"],
                    help="decode mode: v2 (both phases) or v1 (the single-pass entry point)")
    a = ap.parse_args()
    out = os.path.abspath(a.out)
    os.makedirs(out, exist_ok=True)
    steps = a.steps if a.steps is not None else (50 if a.mode == "prefix" else 10)
    trace = kernel_trace(a.config, out, steps, a.mode, a.entry)
    if a.mode == "prefix":
        path = write_prefix_summary(out, trace, pmc(a.config, out, a.mode) if a.pmc else None)
        print(open(path).read(), flush=True)
        return
    counters = pmc(a.config, out, a.mode, a.entry) if a.pmc else None
    if a.mode == "cache_write":
        path = write_cache_summary(a.config, out, trace, counters)
    elif a.mode == "blocksparse":
        path = write_summary(a.config, out, trace, counters, None, "blocksparse")
    else:
        sqv = sq(a.config, out) if a.sq else None
        path = write_summary(a.config, out, trace, counters, sqv, a.entry)
    print(open(path).read(), flush=True)


if __name__ == "__main__":
    main()
