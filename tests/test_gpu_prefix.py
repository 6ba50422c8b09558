"""Paged prefix attention on the GPU (pav2_paged_prefix_attention through the C
ABI) against the oracle.

The chunks' keys and values are first written into the device cache with
pav2_reshape_and_cache (as a backend does before attention); the oracle
reads them from the key / value tensors instead, as the page's fallback does.
Every other cache slot the chunks do not cover holds NaN, so a read of an
unwritten or foreign slot shows up.  Tolerances as for decode: 2e-3 (16-bit)
or one ulp of the output dtype where that is larger, 2e-5 for f32.
"""
import numpy as np
import pytest
import torch

import oracle
import _tol
import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
_CODE = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}
_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TOL = {"f32": 2e-5, "f16": 2e-3, "bf16": 2e-3}


def run_case(ctx, ql, H, KVH, d, BS, dtype, seed=0):
    pw = W.prefix_workload(ctx, ql, H, KVH, d, BS, dtype=dtype, seed=seed)
    scale = d ** -0.5
    ref = oracle.prefix_attention(pw.query, pw.key, pw.value, pw.key_cache, pw.value_cache, pw.block_tables,
                                  pw.query_start_loc, pw.context_lens, num_kv_heads=KVH, block_size=BS,
                                  scale=scale, q_dtype=_CODE[dtype], kv_dtype=_CODE[dtype])
    g = pw.to(DEV)
    pav2.reshape_and_cache(g.key, g.value, g.key_cache, g.value_cache, g.slot_mapping)
    out = torch.full_like(g.query, float("nan"))
    pav2.paged_prefix_attention(out, g.query, g.key_cache, g.value_cache, g.block_tables, g.query_start_loc,
                                g.context_lens, max(ql) if ql else 0, max(c + q for c, q in zip(ctx, ql)),
                                scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), ref


def assert_close(out, ref, dtype):
    got = out.double().numpy()
    assert np.isfinite(got).all()
    return _tol.check(got, ref, _TD[dtype], TOL[dtype], "prefix out")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 80, 96, 112, 120, 128, 192, 256])   # MFMA kernel: 64, 96, 128, 192, 256 (16-bit)
def test_prefix_matches_oracle(dtype, d):
    print(f"case prefix {dtype} d={d}", flush=True)
    # contexts: none, under one tile, one partition, several partitions; chunks of 1 .. 70 tokens, one empty
    ctx, ql = [0, 5, 512, 700, 1100, 33], [7, 1, 16, 33, 70, 0]
    out, ref = run_case(ctx, ql, 12, 2, d, 16, dtype, seed=d)
    assert_close(out, ref, dtype)


@pytest.mark.parametrize("H,KVH", [(4, 4), (8, 1), (24, 4), (32, 1)])
def test_prefix_gqa_row_blocks(H, KVH):
    """Blocks of 16 (token, head) rows that cut across tokens (gqa 6) or hold one head only (gqa 1)."""
    print(f"case prefix gqa H={H} KVH={KVH}", flush=True)
    out, ref = run_case([300, 0, 1030], [21, 40, 9], H, KVH, 128, 16, "bf16", seed=H + KVH)
    assert_close(out, ref, "bf16")


@pytest.mark.parametrize("BS", [1, 2, 4, 8, 32, 64, 512])
def test_prefix_block_sizes(BS):
    print(f"case prefix block {BS}", flush=True)
    out, ref = run_case([17, 600], [30, 12], 8, 2, 64, BS, "bf16", seed=BS)
    assert_close(out, ref, "bf16")


def test_prefix_chunk_longer_than_a_partition():
    """A chunk spanning several partitions: rows' causal limits fall in different partitions."""
    print("case prefix long chunk", flush=True)
    out, ref = run_case([100], [1100], 4, 1, 64, 16, "bf16", seed=9)
    assert_close(out, ref, "bf16")


def test_prefix_medium_gqa6_d256():
    """The long-context layout (24 query heads over 4 kv heads, d = 256, bf16) at a size the oracle finishes."""
    print("case prefix medium", flush=True)
    out, ref = run_case([1500, 700], [96, 40], 24, 4, 256, 16, "bf16", seed=11)
    assert_close(out, ref, "bf16")


def test_prefix_one_token_chunks_match_decode_oracle():
    """One-token chunks are decode steps: compared with the decode oracle on the written cache."""
    pw = W.prefix_workload([37, 600, 0], [1, 1, 1], 6, 2, 128, 16, dtype="bf16", seed=12)
    g = pw.to(DEV)
    pav2.reshape_and_cache(g.key, g.value, g.key_cache, g.value_cache, g.slot_mapping)
    out = torch.full_like(g.query, float("nan"))
    pav2.paged_prefix_attention(out, g.query, g.key_cache, g.value_cache, g.block_tables, g.query_start_loc,
                                g.context_lens, 1, 601)
    kb, vb = oracle.reshape_and_cache(pw.key, pw.value, pw.key_cache, pw.value_cache, pw.slot_mapping,
                                      block_size=16, cache_dtype=oracle.BF16)
    kc = torch.from_numpy(kb).view(torch.bfloat16).reshape(pw.key_cache.shape)
    vc = torch.from_numpy(vb).view(torch.bfloat16).reshape(pw.value_cache.shape)
    ref = oracle.dense_attention(pw.query, kc, vc, pw.block_tables, torch.tensor([38, 601, 1], dtype=torch.int32),
                                 num_kv_heads=2, scale=128 ** -0.5, block_size=16, q_dtype=oracle.BF16,
                                 kv_dtype=oracle.BF16)
    torch.cuda.synchronize()
    assert_close(out.cpu(), ref, "bf16")


def _prefix_call(g, ql, ctx, scale, workspace):
    out = torch.full_like(g.query, float("nan"))
    pav2.paged_prefix_attention(out, g.query, g.key_cache, g.value_cache, g.block_tables, g.query_start_loc,
                                g.context_lens, max(ql), max(c + q for c, q in zip(ctx, ql)), scale=scale,
                                workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("dtype,d,ctx,ql,H,KVH", [
    ("bf16", 256, [3000], [40], 8, 1),               # 3 row blocks over 48 tiles: 8 key ranges
    ("f16", 128, [2100, 0, 64, 900], [30, 50, 1, 7], 12, 4),   # ragged: empty ranges, rows before a range
    ("bf16", 64, [5000, 40], [3, 90], 16, 2),
    ("f16", 192, [2500], [20], 6, 1),                # merge columns not a multiple of the 16-lane step
    ("bf16", 96, [4000, 100], [10, 30], 8, 2),
])
def test_prefix_key_ranges_split(dtype, d, ctx, ql, H, KVH):
    """Few row blocks over long contexts: the call splits each row block's keys
    into ranges merged afterwards.  The split result matches the oracle, the
    unsplit call (workspace None) matches it too, and the two agree to float32
    rounding of the merge."""
    print(f"case prefix split {dtype} d={d} ctx={ctx}", flush=True)
    pw = W.prefix_workload(ctx, ql, H, KVH, d, 16, dtype=dtype, seed=d + len(ctx))
    scale = d ** -0.5
    ref = oracle.prefix_attention(pw.query, pw.key, pw.value, pw.key_cache, pw.value_cache, pw.block_tables,
                                  pw.query_start_loc, pw.context_lens, num_kv_heads=KVH, block_size=16,
                                  scale=scale, q_dtype=_CODE[dtype], kv_dtype=_CODE[dtype])
    g = pw.to(DEV)
    pav2.reshape_and_cache(g.key, g.value, g.key_cache, g.value_cache, g.slot_mapping)
    max_seq = max(c + q for c, q in zip(ctx, ql))
    assert pav2.prefix_workspace_bytes(g.query, g.key_cache, g.value_cache, g.context_lens, max(ql), max_seq,
                                       scale) > 0
    split = _prefix_call(g, ql, ctx, scale, "auto")
    whole = _prefix_call(g, ql, ctx, scale, None)
    assert_close(split, ref, dtype)
    assert_close(whole, ref, dtype)
    # both are the output dtype's rounding of nearly the same float32 value
    diff = (split.double() - whole.double()).abs().max().item()
    assert diff <= 2 * _tol.ulp(np.abs(whole.double().numpy()).max(), _TD[dtype]), diff


def test_prefix_small_workspace_runs_unsplit():
    """A workspace below the query's size is not used: the result is the unsplit call's, bit for bit."""
    ctx, ql = [3000], [40]
    pw = W.prefix_workload(ctx, ql, 8, 1, 128, 16, dtype="bf16", seed=3)
    g = pw.to(DEV)
    pav2.reshape_and_cache(g.key, g.value, g.key_cache, g.value_cache, g.slot_mapping)
    need = pav2.prefix_workspace_bytes(g.query, g.key_cache, g.value_cache, g.context_lens, 40, 3040)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    a = _prefix_call(g, ql, ctx, None, small)
    b = _prefix_call(g, ql, ctx, None, None)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefix_rejects_fp8_cache():
    pw = W.prefix_workload([4], [2], 4, 4, 64, 16, dtype="bf16").to(DEV)
    kc = pw.key_cache.to(torch.float8_e4m3fn)
    with pytest.raises(ValueError):
        pav2.paged_prefix_attention(torch.empty_like(pw.query), pw.query, kc, pw.value_cache, pw.block_tables,
                                    pw.query_start_loc, pw.context_lens, 2, 6)


def test_prefix_full_size_sampled():
    """The benchmark's chunked prefill (4 x (16384 cached + 512 new) tokens, H = 24,
    kv_h = 4, d = 256, bf16), launched as bench.py launches it; sampled rows
    against the oracle.  Row j of a chunk only sees keys up to ctx + j, so it
    is checked as a one-token chunk over the first ctx + j cached tokens, with
    the token's own key and value from the input tensors.  The oracle's cache
    is the generator's starting cache with the chunks written into it by the
    oracle's own cache write (from the key / value tensors): nothing the
    oracle reads comes from the device's cache write."""
    import bench
    c = bench.PREFIX_CASE
    print("case prefix full size", flush=True)
    pw = W.prefix_workload(c["ctx"], c["ql"], c["H"], c["KVH"], c["d"], c["bs"], dtype=c["dtype"], seed=c["seed"],
                           device=DEV)
    host = pw.to("cpu")   # the generator's inputs, taken before the device cache write
    pav2.reshape_and_cache(pw.key, pw.value, pw.key_cache, pw.value_cache, pw.slot_mapping)
    out = torch.full_like(pw.query, float("nan"))
    max_seq = max(a + b for a, b in zip(c["ctx"], c["ql"]))
    pav2.paged_prefix_attention(out, pw.query, pw.key_cache, pw.value_cache, pw.block_tables, pw.query_start_loc,
                                pw.context_lens, max(c["ql"]), max_seq)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    got = out.cpu()
    # every output, not only the sampled rows: a second call is bit-identical
    # (the tiles' hand-off between wavefronts leaves nothing to timing), and
    # the unsplit call agrees to the output dtype's rounding
    again = torch.full_like(pw.query, float("nan"))
    whole = torch.full_like(pw.query, float("nan"))
    pav2.paged_prefix_attention(again, pw.query, pw.key_cache, pw.value_cache, pw.block_tables, pw.query_start_loc,
                                pw.context_lens, max(c["ql"]), max_seq)
    pav2.paged_prefix_attention(whole, pw.query, pw.key_cache, pw.value_cache, pw.block_tables, pw.query_start_loc,
                                pw.context_lens, max(c["ql"]), max_seq, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(again.cpu().view(torch.int16), got.view(torch.int16))
    wd = whole.cpu().double()
    diff = (wd - got.double()).abs().max().item()
    assert diff <= 2 * _tol.ulp(wd.abs().max().item(), torch.bfloat16), diff
    kb, vb = oracle.reshape_and_cache(host.key, host.value, host.key_cache, host.value_cache, host.slot_mapping,
                                      block_size=c["bs"], cache_dtype=oracle.BF16)
    kc = torch.from_numpy(kb).view(torch.bfloat16).reshape(host.key_cache.shape)
    vc = torch.from_numpy(vb).view(torch.bfloat16).reshape(host.value_cache.shape)
    qsl = host.query_start_loc
    worst = 0.0
    for s, j in [(0, 0), (0, 511), (1, 255), (2, 1), (3, 400), (3, 511)]:
        q = int(qsl[s]) + j
        ref = oracle.prefix_attention(host.query[q:q + 1], host.key[q:q + 1], host.value[q:q + 1], kc, vc,
                                      host.block_tables[s:s + 1], torch.tensor([0, 1], dtype=torch.int32),
                                      torch.tensor([c["ctx"][s] + j], dtype=torch.int32), num_kv_heads=c["KVH"],
                                      block_size=c["bs"], scale=c["d"] ** -0.5, q_dtype=oracle.BF16,
                                      kv_dtype=oracle.BF16)
        worst = max(worst, assert_close(got[q:q + 1], ref, "bf16"))
    print(f"  worst {worst:.3g}", flush=True)
