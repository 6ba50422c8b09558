"""Pins for the oracle's block-sparse V2 (CPU only).

The pages name the block-sparse arguments and one rule (the branch is taken
when blocksparse_vert_stride > 1; the sparse block size is a multiple of the
cache block size) but show no body; the reading is stated in
pav2_oracle.c.  The pins check the oracle against things other than its own
predicate: a set-based construction of each head's attended blocks written
here in Python, fed to torch's scaled_dot_product_attention as a boolean
mask over K/V de-paged with torch views; dense decode where the pattern
covers everything; the partitioned == unpartitioned invariant; and
hand-derived means of attended positions (tests/golden).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from _brute import depage, f32
from decode_attention_paged_v2_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make(lens, H=8, KVH=2, D=64, BS=16, q="f32", kv="f32", alibi=False, seed=7, k_scale=1.0, v_scale=1.0):
    spec = W.Spec("bs", H, KVH, D, BS, q, kv, lambda g: list(lens), pool=lambda n: n + 5, alibi=alibi,
                  k_scale=k_scale, v_scale=v_scale, seed=seed)
    return W.generate(spec, poison=True)


def kw(wl, sp=None):
    a = dict(num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
             q_dtype=oracle.dtype_code(wl.q_dtype), kv_dtype=oracle.dtype_code(wl.kv_dtype),
             alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale)
    if sp:
        a.update(tp_rank=sp[0], blocksparse_local_blocks=sp[1], blocksparse_vert_stride=sp[2],
                 blocksparse_block_size=sp[3], blocksparse_head_sliding_step=sp[4])
    return a


def v2(wl, sp=None):
    return oracle.paged_attention_v2(wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.seq_lens,
                                     max_num_partitions=wl.max_num_partitions, **kw(wl, sp))


def dense(wl, sp=None):
    return oracle.dense_attention(wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.seq_lens,
                                  **kw(wl, sp))


def attended_blocks(L, H, tp_rank, local, stride, B, step, h):
    """Set of sparse blocks head h attends: the local window plus the head's stripes."""
    q = (L - 1) // B
    blocks = set(range(max(0, q - local + 1), q + 1))
    hp = tp_rank * H + h
    first = (hp * step) % stride            # Python's % is the mathematical modulo
    blocks |= set(range(first, q + 1, stride))
    return blocks


def masked_sdpa(wl, s, sp):
    """float64 SDPA over the de-paged sequence with the heads' attended tokens as a boolean mask."""
    tp, local, stride, B, step = sp
    L, H, d = int(wl.seq_lens_host[s]), wl.num_heads, wl.head_size
    out = torch.zeros(H, d, dtype=torch.float64)
    if L == 0:
        return out
    k, v = depage(wl, s)
    gqa = H // wl.num_kv_heads
    k = k.permute(1, 0, 2).repeat_interleave(gqa, dim=0)
    v = v.permute(1, 0, 2).repeat_interleave(gqa, dim=0)
    q = wl.query.cpu()[s].to(torch.float64).unsqueeze(1)
    for h in range(H):
        keep = torch.tensor([t // B in attended_blocks(L, H, tp, local, stride, B, step, h) for t in range(L)])
        if not keep.any():
            continue                       # no attended token: zero row
        bias = torch.where(keep, 0.0, -float("inf")).to(torch.float64)
        if wl.alibi_slopes is not None:
            bias = bias + float(wl.alibi_slopes[h]) * torch.arange(L, dtype=torch.float64)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[h:h + 1].unsqueeze(0), k[h:h + 1].unsqueeze(0), v[h:h + 1].unsqueeze(0),
            attn_mask=bias.view(1, 1, 1, L), scale=f32(wl.scale))
        out[h] = o[0, 0, 0]
    return out


@pytest.mark.parametrize("vs", [0, 1])
def test_stride_at_most_one_is_dense(vs):
    wl = make([1, 700, 1300], alibi=True, seed=3)
    r, d = v2(wl, (2, 1, vs, 48, 3)), v2(wl)
    for key in ("out", "max_logits", "exp_sums", "tmp_output"):
        assert np.array_equal(r[key], d[key], equal_nan=True)


def test_window_covering_the_sequence_is_dense():
    wl = make([33, 1030], seed=4)
    r, d = v2(wl, (0, 100, 4, 16, 1)), v2(wl)
    assert np.array_equal(r["out"], d["out"])
    assert np.array_equal(dense(wl, (0, 100, 4, 16, 1)), dense(wl))


SPARSE_CASES = [
    # (tp_rank, local_blocks, vert_stride, sparse block size, sliding step)
    (0, 2, 3, 16, 1),
    (0, 1, 4, 32, 0),
    (1, 3, 5, 48, 2),
    (0, 0, 2, 16, 1),      # no local window: stripes only
    (2, 1, 3, 64, -1),     # negative step
]


@pytest.mark.parametrize("sp", SPARSE_CASES)
@pytest.mark.parametrize("q,kv,alibi", [("f32", "f32", False), ("bf16", "bf16", True), ("f16", "fp8_e4m3", False)])
def test_matches_masked_sdpa(sp, q, kv, alibi):
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    wl = make([1, 17, 300, 513, 1100, 0], H=8, KVH=2, q=q, kv=kv, alibi=alibi, k_scale=ks, v_scale=vs,
              seed=sp[3] + sp[2])
    r = v2(wl, sp)
    for s in range(wl.num_seqs):
        np.testing.assert_allclose(r["out"][s], masked_sdpa(wl, s, sp).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sp", SPARSE_CASES)
def test_partitioned_equals_unpartitioned(sp):
    wl = make([2049, 700, 5], H=6, KVH=3, alibi=True, seed=11)
    r, d = v2(wl, sp), dense(wl, sp)
    np.testing.assert_allclose(r["out"], d, rtol=1e-12, atol=1e-13)


def test_partitions_and_rows_without_attended_tokens():
    # stride 40 over a 1100-token sequence (sparse blocks 0..68 of 16 tokens),
    # no local window: head h' attends only blocks k = 7 h' (mod 40), so the
    # third partition (blocks 64..68) holds none for any head; its statistics
    # must be -inf / 0 with a zero output row, and a head whose stripes miss
    # the whole sequence gets a zero output
    H, sp = 4, (0, 0, 40, 16, 7)
    wl = make([1100, 100], H=H, KVH=1, seed=5)
    r = v2(wl, sp)
    for s, L in enumerate(wl.seq_lens_host):
        for h in range(H):
            blocks = attended_blocks(L, H, *sp[:1], sp[1], sp[2], sp[3], sp[4], h)
            for p in range((L + 511) // 512):
                toks = [t for t in range(512 * p, min(512 * p + 512, L)) if t // 16 in blocks]
                if not toks:
                    assert r["max_logits"][s, h, p] == -np.inf and r["exp_sums"][s, h, p] == 0.0
                    assert np.all(r["tmp_output"][s, h, p] == 0.0)
                else:
                    assert np.isfinite(r["max_logits"][s, h, p]) and r["exp_sums"][s, h, p] > 0
            if not blocks:
                assert np.all(r["out"][s, h] == 0.0)
    # sequence 1 (100 tokens, blocks 0..6): h' = 1, 2, 3 stripe first at 7, 14, 21 -> nothing
    assert [bool(attended_blocks(100, H, 0, 0, 40, 16, 7, h)) for h in range(H)] == [True, False, False, False]
    assert np.all(r["out"][1, 1:] == 0.0) and np.any(r["out"][1, 0] != 0.0)
    ref = masked_sdpa(wl, 0, sp).numpy()
    np.testing.assert_allclose(r["out"][0], ref, rtol=0, atol=1e-12)


def test_rejects_sparse_block_not_a_multiple_of_the_block_size():
    wl = make([40], seed=1)
    with pytest.raises(ValueError):
        v2(wl, (0, 1, 2, 24, 0))


def test_golden_mean_of_attended_positions():
    with open(os.path.join(GOLDEN, "blocksparse_positions.json")) as f:
        g = json.load(f)
    L, BS, D = g["seq_len"], g["block_size"], g["head_size"]
    for c in g["cases"]:
        H = c["num_heads"]
        wl = make([L], H=H, KVH=1, D=D, BS=BS, seed=2)
        wl.scale = g["scale"]
        wl.query.zero_()
        n = (L + BS - 1) // BS
        for t in range(L):
            b = int(wl.block_tables[0, t // BS])
            wl.value_cache[b, 0, :, t % BS] = float(t)
        sp = (c["tp_rank"], c["local_blocks"], c["vert_stride"], c["sparse_block_size"], c["head_sliding_step"])
        for fn in (lambda: v2(wl, sp)["out"], lambda: dense(wl, sp)):
            out = fn()
            for h in range(H):
                want = c["sum"][h] / c["count"][h]
                assert np.all(np.abs(out[0, h] - want) < g["tolerance"]), (c["name"], h, out[0, h, 0], want)
