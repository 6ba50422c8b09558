"""Pins for the oracle's paged prefix attention (CPU only).

Checked against torch's scaled_dot_product_attention in float64 on keys and
values de-paged with torch views (context) and concatenated with the chunk's
own keys and values, under an explicit causal mask; against torch's
is_causal=True when there is no context; against the decode oracle when the
chunk is one token; and against the constant-V closed form.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_v2_amd import workloads as W
from _brute import f32

_CODE = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}


def run(pw, dtype, scale):
    return oracle.prefix_attention(pw.query, pw.key, pw.value, pw.key_cache, pw.value_cache, pw.block_tables,
                                   pw.query_start_loc, pw.context_lens, num_kv_heads=pw.num_kv_heads,
                                   block_size=pw.block_size, scale=scale, q_dtype=_CODE[dtype],
                                   kv_dtype=_CODE[dtype])


def sdpa_ref(pw, s, scale):
    """float64 reference for sequence s: [q_len, H, d]."""
    ctx, ql = pw.ctx_host[s], pw.qlen_host[s]
    q0 = int(pw.query_start_loc[s])
    H, KVH, BS = pw.query.shape[1], pw.num_kv_heads, pw.block_size
    d = pw.query.shape[2]
    n = (ctx + BS - 1) // BS
    blk = pw.block_tables[s, :n].long()
    kc = pw.key_cache[blk].double().permute(0, 3, 1, 2, 4).reshape(-1, KVH, d)[:ctx]
    vc = pw.value_cache[blk].double().permute(0, 3, 1, 2).reshape(-1, KVH, d)[:ctx]
    k = torch.cat([kc, pw.key[q0:q0 + ql].double()])          # [ctx + ql, KVH, d]
    v = torch.cat([vc, pw.value[q0:q0 + ql].double()])
    gqa = H // KVH
    k = k.permute(1, 0, 2).repeat_interleave(gqa, 0)           # [H, n, d]
    v = v.permute(1, 0, 2).repeat_interleave(gqa, 0)
    q = pw.query[q0:q0 + ql].double().permute(1, 0, 2)         # [H, ql, d]
    pos_q = ctx + torch.arange(ql)
    mask = torch.arange(ctx + ql)[None, :] <= pos_q[:, None]   # [ql, ctx + ql]
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None, None],
                                                          scale=f32(scale))
    return o[0].permute(1, 0, 2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ctx,ql,H,KVH,d,BS", [
    ([0, 5, 40], [7, 1, 19], 4, 2, 64, 16),
    ([33, 0], [16, 3], 6, 1, 32, 8),
    ([17], [40], 8, 8, 64, 32),
])
def test_prefix_oracle_matches_masked_sdpa(dtype, ctx, ql, H, KVH, d, BS):
    pw = W.prefix_workload(ctx, ql, H, KVH, d, BS, dtype=dtype, seed=3)
    scale = d ** -0.5
    out = run(pw, dtype, scale)
    for s in range(len(ctx)):
        q0 = int(pw.query_start_loc[s])
        ref = sdpa_ref(pw, s, scale).numpy()
        assert np.max(np.abs(out[q0:q0 + ql[s]] - ref)) < 1e-12


def test_prefix_oracle_without_context_is_causal_attention():
    pw = W.prefix_workload([0], [25], 4, 4, 64, 16, dtype="f32", seed=4)
    out = run(pw, "f32", 0.125)
    q = pw.query.double().permute(1, 0, 2)[None]
    k = pw.key.double().permute(1, 0, 2)[None]
    v = pw.value.double().permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.125)[0].permute(1, 0, 2)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_prefix_oracle_one_token_chunk_is_decode():
    """A one-token chunk equals decode over context + that token, once the
    token's key / value sit in the cache (the cache write's job)."""
    pw = W.prefix_workload([37, 600], [1, 1], 6, 2, 64, 16, dtype="bf16", seed=5)
    out = run(pw, "bf16", 0.125)
    kb, vb = oracle.reshape_and_cache(pw.key, pw.value, pw.key_cache, pw.value_cache, pw.slot_mapping,
                                      block_size=16, cache_dtype=oracle.BF16)
    kc = torch.from_numpy(kb).view(torch.bfloat16).reshape(pw.key_cache.shape)
    vc = torch.from_numpy(vb).view(torch.bfloat16).reshape(pw.value_cache.shape)
    seq_lens = torch.tensor([38, 601], dtype=torch.int32)
    dec = oracle.dense_attention(pw.query, kc, vc, pw.block_tables, seq_lens, num_kv_heads=2, scale=0.125,
                                 block_size=16, q_dtype=oracle.BF16, kv_dtype=oracle.BF16)
    assert np.max(np.abs(out - dec)) < 1e-12


def test_prefix_oracle_constant_values():
    pw = W.prefix_workload([20, 3], [9, 30], 4, 2, 64, 16, dtype="f32", seed=6)
    pw.value.fill_(0.75)
    pw.value_cache.fill_(0.75)    # chunk slots too: they are never read
    out = run(pw, "f32", 0.125)
    assert np.max(np.abs(out - 0.75)) < 1e-14
