"""The entry points are capturable in a HIP graph (they allocate nothing and
never synchronise the host): each is captured once and the graph replayed
several times, with eager work and synchronisations in between, every replay
compared bit for bit with the eager call on the same inputs."""
import numpy as np
import pytest
import torch

import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def replay_and_check(run, outs, eager, replays=3, fill=0xFF):
    """outs are set to `fill` bytes (eager work) before each replay; a write
    that covers only part of an output needs the fill it started from."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # one untimed call on the capture stream first
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for i in range(replays):
        for o in outs:
            o.view(torch.uint8).fill_(fill)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {i} differs"


@pytest.mark.parametrize("name", ["ragged_alibi", "long_gqa", "fp8_kv"])
def test_graph_decode_v2(name):
    wl = W.generate(W.SMALL_SPECS[name]).to(DEV)
    S, H, D, P = wl.num_seqs, wl.num_heads, wl.head_size, wl.max_num_partitions
    out = torch.empty_like(wl.query)
    es = torch.zeros((S, H, P), dtype=torch.float32, device=DEV)
    ml = torch.zeros_like(es)
    tmp = torch.zeros((S, H, P, D), dtype=wl.q_dtype, device=DEV)
    kvdt = "fp8_e4m3" if wl.kv_dtype == torch.float8_e4m3fn else "auto"

    def run():
        pav2.paged_attention_v2(out, es, ml, tmp, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads,
                                wl.scale, wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len,
                                wl.alibi_slopes, kvdt, wl.k_scale, wl.v_scale)
    run()
    torch.cuda.synchronize()
    eager = [out.clone(), es.clone(), ml.clone()]
    replay_and_check(run, [out, es, ml], eager)


def test_graph_decode_v1_and_cache_write():
    wl = W.generate(W.SMALL_SPECS["batched_gqa"]).to(DEV)
    out = torch.empty_like(wl.query)

    def run_v1():
        pav2.paged_attention_v1(out, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads, wl.scale,
                                wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len)
    run_v1()
    torch.cuda.synchronize()
    replay_and_check(run_v1, [out], [out.clone()])

    cw = W.cache_write_workload(W.SMALL_SPECS["fp8_kv"], DEV)
    cw.key_cache.view(torch.uint8).fill_(0)
    cw.value_cache.view(torch.uint8).fill_(0)

    def run_cw():
        pav2.reshape_and_cache(cw.key, cw.value, cw.key_cache, cw.value_cache, cw.slot_mapping, "fp8_e4m3",
                               cw.k_scale, cw.v_scale)
    run_cw()
    torch.cuda.synchronize()
    # the write covers the mapped slots only: replays start from the zeroed caches too
    replay_and_check(run_cw, [cw.key_cache, cw.value_cache], [cw.key_cache.clone(), cw.value_cache.clone()],
                     fill=0)


def test_graph_prefix():
    pw = W.prefix_workload([300, 17], [40, 9], 24, 4, 128, 16, dtype="bf16", seed=5, device=DEV)
    pav2.reshape_and_cache(pw.key, pw.value, pw.key_cache, pw.value_cache, pw.slot_mapping)
    out = torch.empty_like(pw.query)

    def run():
        pav2.paged_prefix_attention(out, pw.query, pw.key_cache, pw.value_cache, pw.block_tables,
                                    pw.query_start_loc, pw.context_lens, 40, 340)
    run()
    torch.cuda.synchronize()
    replay_and_check(run, [out], [out.clone()])


def test_graph_prefix_split_with_workspace():
    """Few row blocks over a long context: the captured call is the split one
    (attention kernel, then the merge) over a workspace allocated beforehand."""
    ctx, ql = [3000], [40]
    pw = W.prefix_workload(ctx, ql, 8, 1, 128, 16, dtype="bf16", seed=11, device=DEV)
    pav2.reshape_and_cache(pw.key, pw.value, pw.key_cache, pw.value_cache, pw.slot_mapping)
    need = pav2.prefix_workspace_bytes(pw.query, pw.key_cache, pw.value_cache, pw.context_lens, 40, 3040)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(pw.query)

    def run():
        pav2.paged_prefix_attention(out, pw.query, pw.key_cache, pw.value_cache, pw.block_tables,
                                    pw.query_start_loc, pw.context_lens, 40, 3040, workspace=ws)
    run()
    torch.cuda.synchronize()
    replay_and_check(run, [out], [out.clone()])


def test_graph_decode_blocksparse():
    wl = W.generate(W.SMALL_SPECS["ragged_alibi"]).to(DEV)
    S, H, D, P = wl.num_seqs, wl.num_heads, wl.head_size, wl.max_num_partitions
    out = torch.empty_like(wl.query)
    es = torch.zeros((S, H, P), dtype=torch.float32, device=DEV)
    ml = torch.zeros_like(es)
    tmp = torch.zeros((S, H, P, D), dtype=wl.q_dtype, device=DEV)

    def run():
        pav2.paged_attention_v2_blocksparse(out, es, ml, tmp, wl.query, wl.key_cache, wl.value_cache,
                                            wl.num_kv_heads, wl.scale, wl.block_tables, wl.seq_lens,
                                            wl.block_size, wl.max_seq_len, wl.alibi_slopes, "auto",
                                            wl.k_scale, wl.v_scale, tp_rank=0, blocksparse_local_blocks=2,
                                            blocksparse_vert_stride=3, blocksparse_block_size=32,
                                            blocksparse_head_sliding_step=1)
    run()
    torch.cuda.synchronize()
    replay_and_check(run, [out, es, ml], [out.clone(), es.clone(), ml.clone()])
