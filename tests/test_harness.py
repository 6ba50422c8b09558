"""Host-side checks of the rocprofv3 summary writers (no GPU, no profiler):
the single-pass summary is priced with that entry point's bytes, the prefix
summary's unique bytes are the hand count of its fixed case, and bench.py
reads traffic back only from summaries taken on the current kernel sources."""
import json
import os

import bench
from decode_attention_paged_v2_amd import accounting, rocprof_harness as H, workloads as W


def _trace(avg_us):
    return {"command": "rocprofv3 ...", "phase1": {"name": "phase1_kernel", "calls": 3, "avg_us": avg_us,
                                                   "min_us": avg_us, "max_us": avg_us}}


def _counters(fetch, write):
    return {"phase1_fetch_bytes": fetch, "phase1_write_bytes": write, "FETCH_SIZE_copy_kib": 1.0,
            "WRITE_SIZE_copy_kib": 1.0, "FETCH_SIZE_scale": 2.0, "WRITE_SIZE_scale": 1.0,
            "FETCH_SIZE_phase1_kib": fetch / 2048, "WRITE_SIZE_phase1_kib": write / 1024}


def test_bench_args_select_entry_and_mode():
    a = H._bench_args("fp8_kv", "decode", 3, 1, "v1")
    assert a[a.index("--entry") + 1] == "v1" and "--mode" not in a
    a2 = H._bench_args("fp8_kv", "decode", 3, 1)   # both phases even where the planner would take V1
    assert a2[a2.index("--entry") + 1] == "v2"
    p = H._bench_args("long_gqa", "prefix", 3, 1)
    assert p[p.index("--mode") + 1] == "prefix"
    assert H._tag("decode", "tiny", "v1") == "decode_v1_tiny" and H._tag("prefix", "tiny", "v2") == "prefix"


def test_v1_summary_uses_single_pass_bytes(tmp_path):
    spec = W.SPECS["tiny"]
    alg = accounting.spec_bytes(spec)
    path = H.write_summary("tiny", str(tmp_path), _trace(10.0), _counters(3.0e6, 5.0e4), None, "v1")
    assert os.path.basename(path) == "v1_tiny.md"
    data = json.load(open(tmp_path / "v1_tiny.json"))
    assert data["entry"] == "v1"
    # the single pass reads what phase 1 reads and writes one row per query head
    assert data["algorithmic"]["phase1"] == alg["v1"]
    assert data["algorithmic"]["phase1_write"] == spec.num_heads * spec.head_size * 4   # f32 rows, one sequence
    assert data["phase1_traffic_bytes"] == 3.0e6 + 5.0e4
    assert abs(data["phase1_achieved_GBps"] - alg["v1"] / 10e-6 / 1e9) < 1e-6


def _prefix_trace(avg_us, merge_us=None):
    t = {"command": "rocprofv3 ...", "prefix": {"name": "prefix_kernel", "calls": 3, "avg_us": avg_us,
                                                "min_us": avg_us, "max_us": avg_us}}
    if merge_us is not None:
        t["prefix_merge"] = {"name": "prefix_merge_kernel", "calls": 3, "avg_us": merge_us, "min_us": merge_us,
                             "max_us": merge_us}
    return t


def _prefix_counters(fetch, write, mfetch=0.0, mwrite=0.0):
    return {"prefix_fetch_bytes": fetch, "prefix_write_bytes": write, "prefix_merge_fetch_bytes": mfetch,
            "prefix_merge_write_bytes": mwrite, "FETCH_SIZE_copy_kib": 1.0, "WRITE_SIZE_copy_kib": 1.0,
            "FETCH_SIZE_scale": 2.0, "WRITE_SIZE_scale": 1.0, "FETCH_SIZE_prefix_kib": fetch / 2048,
            "WRITE_SIZE_prefix_kib": write / 1024}


def test_prefix_summary_unique_bytes(tmp_path):
    H.write_prefix_summary(str(tmp_path), _prefix_trace(3000.0), _prefix_counters(6.0e8, 2.5e7))
    data = json.load(open(tmp_path / "prefix_attention.json"))
    # 4 sequences of 16384 cached + 512 new tokens, kv_h 4, d 256, bf16; 24 query heads
    tokens = 4 * (16384 + 512)
    kv = tokens * 4 * 2 * 256 * 2
    rows = 4 * 512 * 24 * 256 * 2
    tables = 4 * (16384 + 512) // 16
    assert data["unique_read_bytes"] == kv + rows + 4 * tables + 3 * 4 * 4
    assert data["unique_write_bytes"] == rows   # unsplit (no bench line in the log): the output rows
    assert data["traffic_bytes"] == 6.0e8 + 2.5e7
    assert data["key_range_splits"] == 1


def test_prefix_summary_split_call(tmp_path):
    # the bench line in the trace log names the split; the attention kernel then
    # writes the float32 partials (the workspace), and the call's time adds the merge
    ws = 2 * 384 * 128 * 258 * 4
    (tmp_path / "trace_prefix.log").write_text(
        "progress line\n" + json.dumps({"key_range_splits": 2, "workspace_bytes": ws}) + "\n")
    H.write_prefix_summary(str(tmp_path), _prefix_trace(1000.0, 25.0),
                           _prefix_counters(3.1e8, 1.0e8, 1.0e8, 2.5e7))
    data = json.load(open(tmp_path / "prefix_attention.json"))
    assert data["key_range_splits"] == 2 and data["unique_write_bytes"] == ws
    assert data["traffic_bytes"] == 3.1e8 + 1.0e8 and data["merge_traffic_bytes"] == 1.0e8 + 2.5e7
    flops = bench.prefix_flops(**{k: bench.PREFIX_CASE[k] for k in ("ctx", "ql", "H", "d")})
    assert abs(data["achieved_TFLOPs_call"] - flops / 1025e-6 / 1e12) < 1e-6
    text = open(tmp_path / "prefix_attention.md").read()
    assert "prefix_merge_kernel" in text and "Key ranges per row block: 2" in text


def test_prefix_summary_median(tmp_path):
    # a clock transient over the first back-to-back calls raises the average;
    # the summary also reports the rate at the per-dispatch median
    t = _prefix_trace(1200.0, 30.0)
    t["prefix"]["median_us"] = 1000.0
    t["prefix_merge"]["median_us"] = 25.0
    H.write_prefix_summary(str(tmp_path), t)
    data = json.load(open(tmp_path / "prefix_attention.json"))
    flops = bench.prefix_flops(**{k: bench.PREFIX_CASE[k] for k in ("ctx", "ql", "H", "d")})
    assert abs(data["achieved_TFLOPs_median"] - flops / 1000e-6 / 1e12) < 1e-6
    assert abs(data["achieved_TFLOPs_call_median"] - flops / 1025e-6 / 1e12) < 1e-6
    assert abs(data["achieved_TFLOPs"] - flops / 1200e-6 / 1e12) < 1e-6
    assert "| median (µs) |" in open(tmp_path / "prefix_attention.md").read()


def test_bench_reads_traffic_only_for_current_sources():
    # every committed summary names the sources it was taken on; a lookup
    # returns bytes exactly when that hash is the current one
    root = os.path.join(os.path.dirname(__file__), "..", "profiles")
    cur = H.source_hash()
    for cfg in W.SPECS:
        for entry, name in (("v2", f"phase1_{cfg}.json"), ("v1", f"v1_{cfg}.json")):
            path = os.path.join(root, name)
            if not os.path.exists(path):
                continue
            data = json.load(open(path))
            got = bench.measured_traffic(cfg, entry)
            if data.get("source_hash") == cur and "phase1_traffic_bytes" in data:
                assert got == round(data["phase1_traffic_bytes"])
            else:
                assert got is None


def test_source_hash_covers_the_launch_plan(tmp_path, monkeypatch):
    # the planner (schedule, grid, LDS sizing, scale folding) lives in api.hip
    # and the ABI's constants in pav2.h: editing either must invalidate the
    # stored counters, as editing a kernel does
    for mode in ("decode", "prefix", "cache_write"):
        names = [os.path.basename(f) for f in H.KERNEL_SOURCES[mode]]
        assert "api.hip" in names and "pav2.h" in names
    assert any(n.startswith("phase1_") for n in map(os.path.basename, H.KERNEL_SOURCES["decode"]))
    copies = []
    for f in H.KERNEL_SOURCES["decode"]:
        dst = tmp_path / os.path.basename(f)
        dst.write_bytes(open(f, "rb").read())
        copies.append(str(dst))
    monkeypatch.setitem(H.KERNEL_SOURCES, "decode", copies)
    before = H.source_hash("decode")
    api = tmp_path / "api.hip"
    api.write_bytes(api.read_bytes() + b"\n// planner edit\n")
    assert H.source_hash("decode") != before
