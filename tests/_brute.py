"""Brute-force references used only to pin the oracle.

They take a different route from the oracle on purpose: the paged caches are
de-paged with torch views (gather the sequence's blocks, then the permute and
reshape that the page "paged_attention_v2_pytorch.py" uses in its batched KV
gather), elements are widened by torch's own dtype conversions, and attention
is torch's scaled_dot_product_attention in float64 over the whole sequence.
"""
import torch


def f32(v):
    """A Python float rounded to float32, as the C ABI receives it."""
    return float(torch.tensor(v, dtype=torch.float32))


def depage(wl, s):
    """Dense K, V of sequence s as float64 tensors [L, kv_h, d] (torch ops only)."""
    L = int(wl.seq_lens_host[s])
    bs = wl.block_size
    n = (L + bs - 1) // bs
    blk = wl.block_tables[s, :n].long().cpu()
    kc = wl.key_cache.cpu()[blk].to(torch.float64)
    vc = wl.value_cache.cpu()[blk].to(torch.float64)
    kvh, d = wl.num_kv_heads, wl.head_size
    k = kc.permute(0, 3, 1, 2, 4).reshape(-1, kvh, d)[:L] * f32(wl.k_scale)
    v = vc.permute(0, 3, 1, 2).reshape(-1, kvh, d)[:L] * f32(wl.v_scale)
    return k, v


def sdpa_reference(wl, s):
    """softmax(scale * q K^T + alibi) V for every head of sequence s, float64 [H, d]."""
    L = int(wl.seq_lens_host[s])
    H, d = wl.num_heads, wl.head_size
    if L == 0:
        return torch.zeros(H, d, dtype=torch.float64)
    k, v = depage(wl, s)
    gqa = H // wl.num_kv_heads
    k = k.permute(1, 0, 2).repeat_interleave(gqa, dim=0)       # [H, L, d]
    v = v.permute(1, 0, 2).repeat_interleave(gqa, dim=0)
    q = wl.query.cpu()[s].to(torch.float64).unsqueeze(1)       # [H, 1, d]
    mask = None
    if wl.alibi_slopes is not None:
        pos = torch.arange(L, dtype=torch.float64)
        mask = (wl.alibi_slopes.cpu().to(torch.float64)[:, None] * pos[None, :]).unsqueeze(1)
    out = torch.nn.functional.scaled_dot_product_attention(
        q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0),
        attn_mask=None if mask is None else mask.unsqueeze(0),
        scale=f32(wl.scale))
    return out[0, :, 0, :]
