"""Block-sparse V2 (pav2_paged_attention_v2_blocksparse through the C ABI)
against the oracle's block-sparse V2, element by element: the output, the
used partitions' tmp_output rows and statistics (exactly -inf / 0 where a
head attends nothing in a partition), and the unused slots.  Tolerances as
for the dense decode (tests/_tol.py).
"""
import numpy as np
import pytest
import torch

import oracle
import _tol
import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import _binding as B
from decode_attention_paged_v2_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OUT_TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 2e-3}


def sparse_kw(sp):
    return dict(tp_rank=sp[0], blocksparse_local_blocks=sp[1], blocksparse_vert_stride=sp[2],
                blocksparse_block_size=sp[3], blocksparse_head_sliding_step=sp[4])


def run_gpu(wl, sp):
    d = wl.to(DEV)
    S, H, D, P = wl.num_seqs, wl.num_heads, wl.head_size, wl.max_num_partitions
    out = torch.full((S, H, D), float("nan"), dtype=wl.q_dtype, device=DEV)
    es = torch.full((S, H, P), float("nan"), dtype=torch.float32, device=DEV)
    ml = torch.full_like(es, float("nan"))
    tmp = torch.full((S, H, P, D), float("nan"), dtype=wl.q_dtype, device=DEV)
    pav2.paged_attention_v2_blocksparse(
        out, es, ml, tmp, d.query, d.key_cache, d.value_cache, d.num_kv_heads, d.scale, d.block_tables,
        d.seq_lens, d.block_size, d.max_seq_len, alibi_slopes=d.alibi_slopes,
        kv_cache_dtype="fp8_e4m3" if wl.kv_dtype == torch.float8_e4m3fn else "auto",
        k_scale=d.k_scale, v_scale=d.v_scale, **sparse_kw(sp))
    torch.cuda.synchronize()
    return {"out": out.cpu(), "exp_sums": es.cpu(), "max_logits": ml.cpu(), "tmp_output": tmp.cpu()}


def run_oracle(wl, sp, pairs=None):
    return oracle.paged_attention_v2(
        wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.seq_lens, num_kv_heads=wl.num_kv_heads,
        scale=wl.scale, block_size=wl.block_size, max_num_partitions=wl.max_num_partitions,
        q_dtype=oracle.dtype_code(wl.q_dtype), kv_dtype=oracle.dtype_code(wl.kv_dtype),
        alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale, pairs=pairs, **sparse_kw(sp))


def compare(wl, g, r, pairs=None):
    tol0 = 1e-2 if wl.kv_dtype == torch.float8_e4m3fn else OUT_TOL[wl.q_dtype]
    if pairs is None:
        pairs = [(s, h) for s in range(wl.num_seqs) for h in range(wl.num_heads)]
    worst = 0.0
    for s, h in pairs:
        L = wl.seq_lens_host[s]
        P = (L + 511) // 512
        rm, re_ = r["max_logits"][s, h, :P], r["exp_sums"][s, h, :P]
        used = np.isfinite(rm)
        tol = tol0
        if wl.q_dtype == torch.float32 and used.any():
            tol = tol0 + 2.0 ** -21 * np.abs(rm[used]).max()
        extra = 0.0
        if used.any():
            extra = _tol.tmp_rounding_budget(rm[used], re_[used], r["tmp_output"][s, h, :P][used], wl.q_dtype)
        worst = max(worst, _tol.check(g["out"][s, h].double().numpy(), r["out"][s, h], wl.q_dtype, tol,
                                      f"out[{s},{h}] L={L}", extra))
        gm, ge = g["max_logits"][s, h].double().numpy(), g["exp_sums"][s, h].double().numpy()
        assert np.all(gm[P:] == -np.inf) and np.all(ge[P:] == 0.0), f"unused slots of ({s},{h})"
        # partitions where the head attends nothing: exactly -inf / 0 and a zero row
        assert np.all(gm[:P][~used] == -np.inf) and np.all(ge[:P][~used] == 0.0), f"empty partitions of ({s},{h})"
        gt = g["tmp_output"][s, h, :P].double().numpy()
        assert np.all(gt[~used] == 0.0), f"empty partitions' tmp_output of ({s},{h})"
        if used.any():
            em = np.abs(gm[:P][used] - rm[used])
            assert np.all(em <= 1e-3 + 1e-6 * np.abs(rm[used])), f"max_logits[{s},{h}] err {em.max():.3g}"
            ee = np.abs(ge[:P][used] - re_[used]) / re_[used]
            assert np.all(ee <= 1e-4), f"exp_sums[{s},{h}] rel err {ee.max():.3g}"
            _tol.check(gt[used], r["tmp_output"][s, h, :P][used], wl.q_dtype, tol, f"tmp_output[{s},{h}]")
    return worst


def make(lens, H=8, KVH=2, D=128, BS=16, q="bf16", kv="bf16", alibi=False, seed=3):
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    spec = W.Spec("bsp", H, KVH, D, BS, q, kv, lambda g: list(lens), pool=lambda n: n + 7, alibi=alibi,
                  k_scale=ks, v_scale=vs, seed=seed)
    return W.generate(spec, poison=True)


LENS = [0, 1, 17, 300, 513, 1100, 2049, 64]

PATTERNS = [
    # (tp_rank, local_blocks, vert_stride, sparse block size, sliding step)
    (0, 2, 3, 16, 1),
    (0, 1, 4, 32, 0),
    (1, 3, 5, 48, 2),
    (0, 0, 2, 16, 1),      # stripes only
    (2, 1, 3, 64, -1),     # negative step
    (0, 16, 8, 64, 0),     # the benchmark's pattern
]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.name}", flush=True)
    yield


@pytest.mark.parametrize("sp", PATTERNS)
@pytest.mark.parametrize("q,kv,D,alibi", [("bf16", "bf16", 128, False), ("f16", "f16", 80, True),
                                          ("f32", "f32", 64, True), ("bf16", "fp8_e4m3", 256, False),
                                          ("f16", "fp8_e4m3", 112, True), ("bf16", "bf16", 192, True),
                                          ("f16", "f16", 96, False), ("f32", "f32", 120, False)])
def test_blocksparse_matches_oracle(sp, q, kv, D, alibi):
    wl = make(LENS, H=8, KVH=2, D=D, q=q, kv=kv, alibi=alibi, seed=sp[3] + D)
    g = run_gpu(wl, sp)
    compare(wl, g, run_oracle(wl, sp))


@pytest.mark.parametrize("sp", [(0, 2, 3, 16, 1), (0, 1, 4, 64, 0)])
def test_blocksparse_single_sequence_dense_schedule(sp):
    """One sequence runs the dense grid of partition slots (more than one: the compact list)."""
    wl = make([3000], H=12, KVH=2, D=128, alibi=True, seed=9)
    compare(wl, run_gpu(wl, sp), run_oracle(wl, sp))


@pytest.mark.parametrize("H,KVH", [(32, 8), (32, 16)])
def test_blocksparse_many_sequences_compact_classes(H, KVH):
    """20 sequences: one resident round of workgroups, each XCD walking whole
    (kv head, head group) classes (8 and 16 classes)."""
    sp = (1, 2, 3, 32, 1)
    wl = make(LENS + [700, 90, 1536, 0, 33, 2000, 511, 4, 1025, 260, 1700, 3000], H=H, KVH=KVH, D=64, q="f16",
              kv="f16", alibi=True, seed=H + KVH)
    assert wl.num_seqs == 20
    compare(wl, run_gpu(wl, sp), run_oracle(wl, sp))


def test_blocksparse_phase2_two_pairs_per_wavefront():
    """4480 (sequence, head) pairs with short contexts: phase 2 runs two pairs
    per wavefront; with no local window and a stride of 4, short sequences
    leave some heads nothing to attend (zero rows, weight 0 everywhere)."""
    sp = (0, 0, 4, 16, 1)
    g = torch.Generator().manual_seed(77)
    lens = [0 if i % 29 == 3 else int(x) for i, x in enumerate(torch.randint(0, 1500, (140,), generator=g))]
    wl = make(lens, H=32, KVH=8, D=64, q="f16", kv="f16", seed=78)
    plan = pav2.plan(num_seqs=140, num_heads=32, num_kv_heads=8, head_size=64, block_size=16,
                     max_num_partitions=wl.max_num_partitions, query_dtype=B.F16, kv_cache_dtype=B.F16)
    assert plan["phase2_workgroups"] == 4480 // 2 // 4
    compare(wl, run_gpu(wl, sp), run_oracle(wl, sp))


def test_blocksparse_many_heads_per_group():
    """gqa = 20: two 16-head groups per kv head, heads with different stripes in each."""
    sp = (0, 1, 7, 32, 3)
    wl = make([1500, 700], H=40, KVH=2, D=64, seed=12)
    compare(wl, run_gpu(wl, sp), run_oracle(wl, sp))


@pytest.mark.parametrize("BS,B", [(4, 4), (4, 12), (8, 24), (32, 64), (1, 40), (64, 128)])
def test_blocksparse_block_sizes(BS, B):
    sp = (0, 2, 3, B, 1)
    wl = make([5, 300, 1100], H=6, KVH=2, D=64, BS=BS, seed=BS + B)
    compare(wl, run_gpu(wl, sp), run_oracle(wl, sp))


def test_blocksparse_heads_with_no_attended_token():
    """No local window and stripes every 40 sparse blocks from 7 h': most heads of
    a 100-token sequence attend nothing (zero rows), and the last partition of
    a 1100-token one holds no attended token for any head."""
    sp = (0, 0, 40, 16, 7)
    wl = make([1100, 100], H=4, KVH=1, D=64, seed=5)
    g = run_gpu(wl, sp)
    compare(wl, g, run_oracle(wl, sp))
    assert torch.all(g["out"][1, 1:] == 0)


@pytest.mark.parametrize("vs", [0, 1])
def test_blocksparse_stride_at_most_one_is_the_dense_call(vs):
    wl = make([1, 700, 1300], H=8, KVH=2, D=128, alibi=True, seed=4)
    g = run_gpu(wl, (3, 5, vs, 48, 2))
    d = wl.to(DEV)
    out, es, ml, tmp = pav2.decode(d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, d.num_kv_heads,
                                   d.scale, d.block_size, d.max_seq_len, alibi_slopes=d.alibi_slopes)
    torch.cuda.synchronize()
    assert torch.equal(g["out"].view(torch.int16), out.cpu().view(torch.int16))
    assert torch.equal(g["exp_sums"], es.cpu())


def test_blocksparse_rejects_bad_arguments():
    wl = make([40], seed=1).to(DEV)
    S, H, D, P = wl.num_seqs, wl.num_heads, wl.head_size, wl.max_num_partitions
    out = torch.empty_like(wl.query)
    es = torch.empty((S, H, P), dtype=torch.float32, device=DEV)
    tmp = torch.empty((S, H, P, D), dtype=wl.q_dtype, device=DEV)
    for bad in ((0, 1, 4, 24, 0), (0, 1, 4, 0, 0), (0, -1, 4, 32, 0), (-1, 1, 4, 32, 0)):
        with pytest.raises(pav2.Pav2Error) as e:
            pav2.paged_attention_v2_blocksparse(out, es, es.clone(), tmp, wl.query, wl.key_cache, wl.value_cache,
                                                wl.num_kv_heads, wl.scale, wl.block_tables, wl.seq_lens,
                                                wl.block_size, wl.max_seq_len, **sparse_kw(bad))
        assert e.value.status == -1


def test_blocksparse_full_size_sampled():
    """The benchmark's block-sparse decode: long_gqa (4 x 100000 tokens, H 24,
    kv_h 4, d 256, bf16) with sparse blocks of 64 tokens, a 16-block local
    window and every 8th block; sampled (sequence, head) pairs against the oracle."""
    import bench
    sp = bench.BLOCKSPARSE_PATTERN
    wl = W.generate(W.SPECS["long_gqa"], device=DEV, poison=False)
    g = run_gpu(wl, sp)
    host = wl.to("cpu")
    pairs = [(0, 0), (0, 23), (1, 7), (2, 12), (3, 5), (3, 18)]
    r = run_oracle(host, sp, pairs=pairs)
    worst = compare(host, g, r, pairs)
    print(f"  worst {worst:.3g}", flush=True)
