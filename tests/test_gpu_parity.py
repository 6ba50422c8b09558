"""Parity of the HIP path (called through the C ABI) with the float64 oracle.

Tolerances (max-abs error against the oracle's float64 result rounded to the
output dtype): 2e-3 for f16/bf16 outputs, 1e-2 with an fp8 e4m3 KV cache,
1e-5 (+ 2^-21 max|m_p|, the float32 rounding of the stored max logits) for
f32 -- or one unit in the last place of the output dtype where that
unit is larger (bf16 outputs of magnitude >= 0.5), the least difference two
rounded results can have.  The statistics: max_logits within 1e-3 + 1e-6 |ref|,
exp_sums within 1e-4 relative; unused partition slots must hold exactly
-inf / 0.  Block-table indexing is checked bit-exactly by one-hot probes.
"""
import math
import os
import sys

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
FP8_TOL = 1e-2
GUARD = 4096          # sentinel elements after every output buffer
SENTINEL = 4096.0     # exactly representable in f32, f16 and bf16


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol_for(wl):
    return FP8_TOL if wl.kv_dtype == torch.float8_e4m3fn else OUT_TOL[wl.q_dtype]


def _guarded(shape, dtype, fill):
    n = int(np.prod(shape))
    buf = torch.full((n + GUARD,), fill, dtype=dtype, device=DEV)
    return buf, buf[:n].view(shape)


def run_gpu(wl, stream=None, split=False):
    """Both phases through the C ABI into NaN-filled, sentinel-guarded buffers."""
    S, H, D, P = wl.num_seqs, wl.num_heads, wl.head_size, wl.max_num_partitions
    ob, out = _guarded((S, H, D), wl.q_dtype, float("nan"))
    eb, es = _guarded((S, H, P), torch.float32, float("nan"))
    mb, ml = _guarded((S, H, P), torch.float32, float("nan"))
    tb, tmp = _guarded((S, H, P, D), wl.q_dtype, float("nan"))
    for buf, n in ((ob, out.numel()), (eb, es.numel()), (mb, ml.numel()), (tb, tmp.numel())):
        buf[n:] = SENTINEL
    args = (wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads, wl.scale, wl.block_tables,
            wl.seq_lens, wl.block_size, wl.max_seq_len)
    kw = dict(alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale, stream=stream)
    if split:
        pav2.phase1(es, ml, tmp, *args, **kw)
        pav2.phase2(out, es, ml, tmp, wl.seq_lens, stream=stream)
    else:
        pav2.paged_attention_v2(out, es, ml, tmp, *args, **kw)
    torch.cuda.synchronize()
    for buf, n, name in ((ob, out.numel(), "output"), (eb, es.numel(), "exp_sums"),
                         (mb, ml.numel(), "max_logits"), (tb, tmp.numel(), "tmp_output")):
        assert torch.all(buf[n:].float() == SENTINEL), f"write past the end of {name}"
    return {"out": out.cpu(), "exp_sums": es.cpu(), "max_logits": ml.cpu(), "tmp_output": tmp.cpu()}


def run_oracle(wl, pairs=None):
    return oracle.paged_attention_v2(
        wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.seq_lens,
        num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
        max_num_partitions=wl.max_num_partitions, q_dtype=oracle.dtype_code(wl.q_dtype),
        kv_dtype=oracle.dtype_code(wl.kv_dtype), alibi_slopes=wl.alibi_slopes,
        k_scale=wl.k_scale, v_scale=wl.v_scale, pairs=pairs)


def compare(wl, g, r, pairs=None):
    """Element-by-element check of the GPU result g against the oracle r."""
    tol = tol_for(wl)
    if pairs is None:
        pairs = [(s, h) for s in range(wl.num_seqs) for h in range(wl.num_heads)]
    worst = {"out": 0.0, "tmp": 0.0, "ml": 0.0, "es": 0.0}
    for s, h in pairs:
        L = wl.seq_lens_host[s]
        P = (L + 511) // 512
        go = g["out"][s, h].double().numpy()
        if wl.q_dtype == torch.float32 and P:
            # max_logits are stored as float32 in the pages' absolute frame, so
            # each carries up to 2^-24 |m_p| of rounding into phase 2's weights
            tol = OUT_TOL[torch.float32] + 2.0 ** -21 * np.abs(r["max_logits"][s, h, :P]).max()
        extra = 0.0
        if P:
            extra = _tol.tmp_rounding_budget(r["max_logits"][s, h, :P], r["exp_sums"][s, h, :P],
                                             r["tmp_output"][s, h, :P], wl.q_dtype)
        worst["out"] = max(worst["out"], _tol.check(go, r["out"][s, h], wl.q_dtype, tol, f"out[{s},{h}] L={L}",
                                                     extra=extra))
        gm, ge = g["max_logits"][s, h].double().numpy(), g["exp_sums"][s, h].double().numpy()
        rm, re_ = r["max_logits"][s, h], r["exp_sums"][s, h]
        assert np.all(gm[P:] == -np.inf), f"max_logits[{s},{h},{P}:] not -inf"
        assert np.all(ge[P:] == 0.0), f"exp_sums[{s},{h},{P}:] not 0"
        if P:
            em = np.abs(gm[:P] - rm[:P])
            assert np.all(em <= 1e-3 + 1e-6 * np.abs(rm[:P])), f"max_logits[{s},{h}] err {em.max():.3g}"
            ee = np.abs(ge[:P] - re_[:P]) / re_[:P]
            assert np.all(ee <= 1e-4), f"exp_sums[{s},{h}] rel err {ee.max():.3g}"
            gt = g["tmp_output"][s, h, :P].double().numpy()
            et = _tol.check(gt, r["tmp_output"][s, h, :P], wl.q_dtype, tol, f"tmp_output[{s},{h}]")
            worst["ml"] = max(worst["ml"], em.max())
            worst["es"] = max(worst["es"], ee.max())
            worst["tmp"] = max(worst["tmp"], et)
    return worst


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu case] {request.node.name}")
    yield


# ---- the five workloads at oracle-sized scale, every (seq, head) pair ----------

@pytest.mark.parametrize("name", list(W.SMALL_SPECS))
def test_parity_small(name):
    wl = W.generate(W.SMALL_SPECS[name], poison=True)
    g = run_gpu(wl.to(DEV))
    r = run_oracle(wl)
    worst = compare(wl, g, r)
    say(f"  {name}: worst {worst}")


# ---- the five workloads at full size, sampled pairs -----------------------------

def _sample_pairs(wl, n=14, seed=0):
    rng = np.random.default_rng(seed)
    S, H = wl.num_seqs, wl.num_heads
    n = min(n, S * H)
    pairs = {(0, 0), (S - 1, H - 1), (0, H - 1), (S - 1, 0)}
    lens = wl.seq_lens_host
    pairs.add((int(np.argmax(lens)), int(rng.integers(H))))
    for s in (i for i, L in enumerate(lens) if L in (0, 1)):
        pairs.add((s, int(rng.integers(H))))
    while len(pairs) < n:
        pairs.add((int(rng.integers(S)), int(rng.integers(H))))
    return sorted(pairs)


@pytest.mark.parametrize("name", list(W.SPECS))
def test_parity_full_size_sampled(name):
    spec = W.SPECS[name]
    wl_dev = W.generate(spec, device=DEV, poison=False)
    say(f"  generated {name}: seqs={wl_dev.num_seqs} kv_bytes={wl_dev.kv_bytes() / 1e9:.3f} GB")
    g = run_gpu(wl_dev)
    wl = wl_dev.to("cpu")
    del wl_dev
    torch.cuda.empty_cache()
    pairs = _sample_pairs(wl)
    r = run_oracle(wl, pairs=pairs)
    worst = compare(wl, g, r, pairs)
    # every row is finite and every unused slot is -inf / 0, also off the sample
    assert torch.isfinite(g["out"].float()).all()
    for s, L in enumerate(wl.seq_lens_host):
        P = (L + 511) // 512
        assert torch.all(g["max_logits"][s, :, P:] == -math.inf)
        assert torch.all(g["exp_sums"][s, :, P:] == 0)
    say(f"  {name}: {len(pairs)} pairs, worst {worst}")


# ---- bit-exact probes -------------------------------------------------------------

@pytest.mark.parametrize("kv,q,BS", [("f16", "f16", 16), ("bf16", "bf16", 8), ("f32", "f32", 8),
                                     ("fp8_e4m3", "bf16", 32), ("fp8_e4m3", "f16", 64),
                                     ("bf16", "bf16", 128), ("fp8_e4m3", "f32", 16),
                                     ("f16", "f16", 1), ("fp8_e4m3", "bf16", 2), ("f32", "f32", 4),
                                     ("bf16", "bf16", 4)])
def test_block_table_one_hot_probe(kv, q, BS):
    """Sequence s has K = 0 except its token tau = s, where K[tau, 0] = c with
    scale * c = 200 (q = e_0): the softmax weight of every other token underflows
    to 0 in float32, so the output must be V[tau] bit-exactly (V rows distinct
    per token).  tau sweeps every token of a 3-partition sequence, one sequence
    per tau, each with its own shuffled blocks."""
    L = 2 * 512 + 37
    H, KVH, D = 2, 1, 64
    spec = W.Spec("probe", H, KVH, D, BS, q, kv, lambda g: [L] * L, pool=lambda n: n + 7, seed=BS)
    wl = W.generate(spec, poison=True)
    n = (L + BS - 1) // BS
    wl.query.zero_()
    wl.query[:, :, 0] = 1.0
    c = 448.0 if kv == "fp8_e4m3" else 16.0
    wl.scale = 200.0 / c
    t = torch.arange(n * BS)
    vals = (torch.arange(D)[:, None] % 13 + (t[None, :] % 11) * 0.25 - 2.0).to(torch.float32)
    vpat = vals.reshape(D, n, BS).permute(1, 0, 2).unsqueeze(1).to(wl.kv_dtype)   # [n, 1, D, BS]
    for s in range(L):
        blocks = wl.block_tables[s, :n].long()
        wl.key_cache[blocks] = 0.0
        wl.value_cache[blocks] = vpat
        b = int(wl.block_tables[s, s // BS])
        wl.key_cache[b, 0, 0, s % BS, 0] = c
    g = run_gpu(wl.to(DEV))
    want = vpat.permute(1, 2, 0, 3).reshape(D, n * BS)[:, :L].to(torch.float64).to(wl.q_dtype)
    for s in range(L):
        for h in range(H):
            assert torch.equal(g["out"][s, h], want[:, s]), f"tau={s}: wrong row selected"
        P = (s // 512)
        assert torch.equal(g["tmp_output"][s, 0, P], want[:, s])
        assert float(g["exp_sums"][s, 0, P]) == 1.0


def test_head_dim_probe():
    """q = e_i, K[tau, i] = c: pins the (i // x, i % x) placement of every head-dim
    index in the key cache, bit-exactly."""
    for q, kv in (("f16", "f16"), ("bf16", "fp8_e4m3"), ("f32", "f32")):
        D, BS, L = 128, 16, 40
        spec = W.Spec("dprobe", D, 1, D, BS, q, kv, lambda g: [L], pool=lambda n: n + 3, seed=5)
        wl = W.generate(spec, poison=True)   # one query head per head-dim index
        x = W.x_pack(wl.kv_dtype)
        n = (L + BS - 1) // BS
        blocks = wl.block_tables[0, :n].long()
        wl.key_cache[blocks] = 0.0
        wl.query.zero_()
        c = 448.0 if kv == "fp8_e4m3" else 16.0
        wl.scale = 200.0 / c
        for t in range(L):
            bb = int(wl.block_tables[0, t // BS])
            wl.value_cache[bb, 0, :, t % BS] = float(t % 17)
        for i in range(D):
            tau = (7 * i + 3) % L
            wl.query[0, i, i] = 1.0
            b = int(wl.block_tables[0, tau // BS])
            wl.key_cache[b, 0, i // x, tau % BS, i % x] = c
        g = run_gpu(wl.to(DEV))
        for i in range(D):
            tau = (7 * i + 3) % L
            assert torch.all(g["out"][0, i].float() == float(tau % 17)), f"{q}/{kv} head-dim {i}"


@pytest.mark.parametrize("H,KVH", [(8, 8), (12, 2), (24, 4), (64, 8), (32, 2), (48, 1), (40, 2)])
def test_gqa_mapping_probe(H, KVH):
    """V constant per kv head (= g + 1): query head h must read kv head h // gqa,
    also when gqa > 16 splits a kv head's query heads over several workgroups."""
    spec = W.Spec("gqa", H, KVH, 64, 16, "bf16", "bf16", lambda g: [700, 33, 1024],
                  pool=lambda n: n + 5, seed=H)
    wl = W.generate(spec, poison=True)
    for s, L in enumerate(wl.seq_lens_host):
        n = (L + 15) // 16
        for g in range(KVH):
            for j in range(n):
                b = int(wl.block_tables[s, j])
                upto = min(16, L - 16 * j)
                wl.value_cache[b, g, :, :upto] = float(g + 1)
    g = run_gpu(wl.to(DEV))
    gqa = H // KVH
    for h in range(H):
        assert torch.all(g["out"][:, h].float() == float(h // gqa + 1)), f"head {h}"


# ---- edge sweeps ------------------------------------------------------------------

EDGE_LENS = [0, 1, 2, 15, 16, 17, 511, 512, 513, 1000, 1536, 0, 2049]


@pytest.mark.parametrize("q,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                  ("f32", "fp8_e4m3"), ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("D", [64, 80, 96, 112, 120, 128, 192, 256])
def test_edge_dtypes_head_sizes(q, kv, D):
    if kv == "fp8_e4m3" and D % 16:
        pytest.skip("head size not a multiple of 16 fp8 elements")
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    spec = W.Spec(f"edge_{q}_{kv}_{D}", 6, 2, D, 16, q, kv, lambda g: EDGE_LENS,
                  pool=lambda n: n + 9, alibi=(D % 32 == 16), k_scale=ks, v_scale=vs, seed=D)
    wl = W.generate(spec, poison=True)
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


CLASS_LENS = [0, 1, 700, 513, 2049, 31, 512, 1536, 0, 90, 1100, 3000, 17, 1025, 64, 2000, 511, 4, 1700, 260]


@pytest.mark.parametrize("H,KVH,q,kv", [
    (32, 8, "f16", "f16"),           # 8 (kv head, group) classes: one per XCD
    (32, 16, "bf16", "bf16"),        # 16 classes: two per XCD
    (80, 4, "f16", "f16"),           # 4 kv heads x 2 head groups of 20 query heads
    (64, 8, "bf16", "fp8_e4m3"),
    (24, 12, "f16", "f16"),          # 12 classes: one round, items in order
])
def test_many_sequences_compact_classes(H, KVH, q, kv):
    """20 ragged sequences (empty ones included): the compact grid is one
    resident round and, where the classes are a multiple of 8, each XCD walks
    whole (kv head, head group) classes."""
    plan = pav2.plan(num_seqs=len(CLASS_LENS), num_heads=H, num_kv_heads=KVH, head_size=64, block_size=16,
                     max_num_partitions=6, query_dtype=B.F16, kv_cache_dtype=B.F16)
    assert plan["phase1_rounds"] == 1
    assert plan["phase1_xcd_classes"] == (1 if (KVH * plan["head_groups"]) % 8 == 0 else 0)
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    spec = W.Spec(f"classes_{H}_{KVH}", H, KVH, 64, 16, q, kv, lambda g: CLASS_LENS, pool=lambda n: n + 5,
                  alibi=True, k_scale=ks, v_scale=vs, seed=H + KVH)
    wl = W.generate(spec, poison=True)
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


@pytest.mark.parametrize("S,H,KVH,D,q,kv", [
    (1367, 3, 1, 80, "f16", "f16"),          # 4101 pairs (odd): the last wavefront holds one pair
    (130, 32, 8, 128, "bf16", "bf16"),       # 4160 pairs
    (1100, 4, 2, 64, "f32", "f32"),          # f32 rows of 16 lanes
    (140, 32, 4, 256, "bf16", "fp8_e4m3"),   # a 32-lane row: one group per pair
])
def test_phase2_two_pairs_per_wavefront(S, H, KVH, D, q, kv):
    """More (sequence, head) pairs than one resident round of wavefronts, short
    contexts: phase 2 runs two pairs per wavefront.  Every pair is checked,
    with empty sequences, one-partition and several-partition ones mixed."""
    plan = pav2.plan(num_seqs=S, num_heads=H, num_kv_heads=KVH, head_size=D, block_size=16,
                     max_num_partitions=4, query_dtype=B.F16, kv_cache_dtype=B.F16)
    assert plan["phase2_workgroups"] == -(-(-(-S * H // 2)) // 4)
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    # every 97th sequence empty and every 89th a single token, the rest random
    lens = lambda g: [0 if i % 97 == 5 else (1 if i % 89 == 7 else int(x))
                      for i, x in enumerate(torch.randint(0, 2000, (S,), generator=g))]
    spec = W.Spec(f"p2pairs_{S}_{H}", H, KVH, D, 16, q, kv, lens, pool=lambda n: n + 5, alibi=(D == 80),
                  k_scale=ks, v_scale=vs, seed=S + H)
    wl = W.generate(spec, poison=True)
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


@pytest.mark.parametrize("BS", [1, 2, 4, 8, 32, 64, 128, 256, 512])
def test_edge_block_sizes(BS):
    spec = W.Spec(f"bs{BS}", 8, 2, 128, BS, "f16", "f16", lambda g: [1, max(BS - 1, 0), BS, BS + 1, 1300, 0, 7],
                  pool=lambda n: n + 3, alibi=True, seed=BS)
    wl = W.generate(spec, poison=True)
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


@pytest.mark.parametrize("q,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                  ("f32", "fp8_e4m3"), ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("BS", [1, 2, 4])
def test_small_blocks_every_dtype_pair(q, kv, BS):
    """Blocks of 1, 2 or 4 tokens (the pages only ask that the block size divide
    the 512-token partition): a lane's 8-token V slice then spans several
    blocks.  Ragged lengths across partitions, ALiBi, a non-power-of-two head size."""
    D = 112
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    spec = W.Spec(f"small_{q}_{kv}_{BS}", 8, 2, D, BS, q, kv, lambda g: [0, 1, 3, 9, 511, 513, 1100],
                  pool=lambda n: n + 9, alibi=True, k_scale=ks, v_scale=vs, seed=100 + BS)
    wl = W.generate(spec, poison=True)
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


def test_all_sequences_empty():
    spec = W.Spec("empty", 8, 2, 64, 16, "bf16", "bf16", lambda g: [0, 0, 0], pool=lambda n: 4, seed=1)
    wl = W.generate(spec, poison=True)
    wl.max_seq_len = 0
    g = run_gpu(wl.to(DEV))
    assert torch.all(g["out"] == 0)
    assert torch.all(g["max_logits"] == -math.inf)
    assert torch.all(g["exp_sums"] == 0)


def test_spare_partition_slots_and_inflated_max_seq_len():
    """max_seq_len (and so max_num_partitions) larger than every sequence, as
    with graph-captured batches: extra slots are -inf / 0 and results unchanged."""
    spec = W.SMALL_SPECS["batched_gqa"]
    wl = W.generate(spec, poison=True)
    wl.max_seq_len = 20000
    wl.max_num_partitions = 40
    pad = torch.full((wl.num_seqs, (20000 + 15) // 16), -1, dtype=torch.int32)
    pad[:, :wl.block_tables.shape[1]] = wl.block_tables
    wl.block_tables = pad
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


def test_dense_schedule_for_large_batches_with_spare_slots():
    """Batches of more than 8192 sequences run on the dense grid (one
    workgroup per partition slot); an inflated max_seq_len leaves most slots
    past their sequence's end."""
    n = 8193
    spec = W.Spec("many", 4, 2, 64, 16, "f16", "f16",
                  lambda g: [1300, 600, 0] + torch.randint(0, 40, (n - 3,), generator=g).tolist(),
                  alibi=True, seed=21)
    wl = W.generate(spec, poison=True)
    plan = pav2.plan(n, 4, 2, 64, 16, 6, pav2.F16, pav2.F16)
    assert plan["phase1_compact"] == 0
    wl.max_seq_len = 3000
    wl.max_num_partitions = 6
    pad = torch.full((n, 188), -1, dtype=torch.int32)
    pad[:, :wl.block_tables.shape[1]] = wl.block_tables
    wl.block_tables = pad
    g = run_gpu(wl.to(DEV))
    rng = np.random.default_rng(5)
    pairs = sorted({(0, h) for h in range(4)} | {(1, 3), (2, 0), (n - 1, 2)} |
                   {(int(a), int(b)) for a, b in zip(rng.integers(0, n, 300), rng.integers(0, 4, 300))})
    compare(wl, g, run_oracle(wl, pairs=pairs), pairs=pairs)


# Batches with many partition slots (an inflated max_seq_len: most slots lie
# past their sequence's end) and ragged lengths, across dtypes and head
# sizes, at sizes the oracle covers completely.
MANY_SLOT_CASES = [
    ("f16", "f16", 32, 8, 80, 16, True),
    ("bf16", "fp8_e4m3", 64, 8, 128, 32, False),
    ("bf16", "bf16", 24, 4, 256, 16, False),
    ("f32", "f32", 8, 8, 64, 16, True),
    ("f16", "f16", 16, 2, 120, 8, False),
]


@pytest.mark.parametrize("qd,kvd,H,KVH,d,bs,alibi", MANY_SLOT_CASES)
def test_many_partition_slots(qd, kvd, H, KVH, d, bs, alibi):
    n = 64
    maxP = -(-12288 // (n * KVH * max(1, -(-(H // KVH) // 16))))
    lens = lambda g: [0, 1, 511, 512, 513, 2047, 2600] + torch.randint(1, 2600, (n - 7,), generator=g).tolist()
    spec = W.Spec("slots", H, KVH, d, bs, qd, kvd, lens, alibi=alibi, seed=31,
                  k_scale=0.05 if kvd == "fp8_e4m3" else 1.0, v_scale=0.04 if kvd == "fp8_e4m3" else 1.0)
    wl = W.generate(spec, poison=True)
    wl.max_seq_len = maxP * 512
    wl.max_num_partitions = maxP
    mbps = -(-wl.max_seq_len // bs)
    pad = torch.full((n, mbps), -1, dtype=torch.int32)
    pad[:, :wl.block_tables.shape[1]] = wl.block_tables
    wl.block_tables = pad
    g = run_gpu(wl.to(DEV))
    worst = compare(wl, g, run_oracle(wl))
    say(f"  worst {worst}")


def test_single_sequence_dense_schedule_with_spare_slots():
    """One sequence runs on the dense grid (one workgroup per partition slot);
    an inflated max_seq_len makes most slots start past the sequence end."""
    spec = W.Spec("single", 16, 2, 128, 16, "bf16", "bf16", lambda g: [1300], pool=lambda n: n + 3,
                  alibi=True, seed=9)
    wl = W.generate(spec, poison=True)
    plan = pav2.plan(1, 16, 2, 128, 16, 20, pav2.BF16, pav2.BF16)
    assert plan["phase1_compact"] == 0
    wl.max_seq_len = 10000
    wl.max_num_partitions = 20
    pad = torch.full((1, 625), -1, dtype=torch.int32)
    pad[:, :wl.block_tables.shape[1]] = wl.block_tables
    wl.block_tables = pad
    g = run_gpu(wl.to(DEV))
    compare(wl, g, run_oracle(wl))


def test_split_phases_match_single_call_and_are_deterministic():
    wl = W.generate(W.SMALL_SPECS["ragged_alibi"], poison=True).to(DEV)
    a = run_gpu(wl)
    b = run_gpu(wl, split=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = run_gpu(wl, stream=s)
    for k in a:
        assert torch.equal(a[k].nan_to_num(7.0), b[k].nan_to_num(7.0)), k
        assert torch.equal(a[k].nan_to_num(7.0), c[k].nan_to_num(7.0)), k


def test_constant_value_rows():
    spec = W.Spec("const", 12, 4, 80, 16, "f16", "f16", lambda g: [1, 600, 1501],
                  pool=lambda n: n + 2, alibi=True, seed=3)
    wl = W.generate(spec, poison=False)
    wl.value_cache.fill_(1.5)
    g = run_gpu(wl.to(DEV))
    assert torch.all(g["out"].float() == 1.5)


# ---- device element decoding --------------------------------------------------------

@pytest.mark.parametrize("via", [torch.float32, torch.float16, torch.bfloat16])
def test_decode_fp8_all_codes(via):
    codes = torch.arange(256, dtype=torch.uint8)
    src = codes.view(torch.float8_e4m3fn).to(DEV)
    got = pav2.decode_kv(src, compute_dtype=via).cpu()
    ref = codes.view(torch.float8_e4m3fn).float()
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_decode_16bit_all_codes(dt):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    src = codes.view(dt).to(DEV)
    got = pav2.decode_kv(src).cpu()
    ref = codes.view(dt).float()
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], ref[~nan])
