"""Parity of the single-pass (V1) entry point with the float64 oracle.

V1 computes the same attention as V2 in one launch (page "paged_attn.py",
forward_decode, chooses between them), so its reference is the oracle's
unpartitioned softmax (oracle.dense_attention), with the output tolerances of
the V2 tests: 2e-3 for f16/bf16 outputs, 1e-2 with an fp8 e4m3 KV cache, and
for f32 1e-5 + 2^-21 max|m_p| (the running maximum is carried in float32 in
the absolute-position frame), or one unit in the last place of the output
dtype where that is larger.  Indexing is checked bit-exactly by one-hot
probes; the planner's V1/V2 choice and the dispatching entry point are
checked against the same oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import _tol
import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OUT_TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 2e-3}
FP8_TOL = 1e-2
GUARD = 4096
SENTINEL = 4096.0


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu case] {request.node.name}")
    yield


def run_v1(wl, stream=None):
    """The V1 entry point through the C ABI into a NaN-filled, sentinel-guarded buffer."""
    S, H, D = wl.num_seqs, wl.num_heads, wl.head_size
    n = S * H * D
    buf = torch.full((n + GUARD,), float("nan"), dtype=wl.q_dtype, device=DEV)
    buf[n:] = SENTINEL
    out = buf[:n].view(S, H, D)
    pav2.paged_attention_v1(out, wl.query, wl.key_cache, wl.value_cache, wl.num_kv_heads, wl.scale,
                            wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len,
                            alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale,
                            stream=stream)
    torch.cuda.synchronize()
    assert torch.all(buf[n:].float() == SENTINEL), "write past the end of output"
    return out.cpu()


def oracle_kw(wl):
    return dict(num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
                q_dtype=oracle.dtype_code(wl.q_dtype), kv_dtype=oracle.dtype_code(wl.kv_dtype),
                alibi_slopes=wl.alibi_slopes, k_scale=wl.k_scale, v_scale=wl.v_scale)


def run_dense(wl, pairs=None):
    return oracle.dense_attention(wl.query, wl.key_cache, wl.value_cache, wl.block_tables,
                                  wl.seq_lens, pairs=pairs, **oracle_kw(wl))


def max_abs_logit(wl, pairs):
    """max |m_p| over the pairs' partitions (the oracle's partition maxima)."""
    r = oracle.paged_attention_v2(wl.query, wl.key_cache, wl.value_cache, wl.block_tables,
                                  wl.seq_lens, max_num_partitions=wl.max_num_partitions,
                                  pairs=pairs, **oracle_kw(wl))
    ml = r["max_logits"]
    return {(s, h): float(np.abs(ml[s, h][np.isfinite(ml[s, h])]).max(initial=0.0)) for s, h in pairs}


def compare(wl, go, ro, pairs=None):
    """Element-by-element check of the V1 output against the dense oracle."""
    if pairs is None:
        pairs = [(s, h) for s in range(wl.num_seqs) for h in range(wl.num_heads)]
    tol = FP8_TOL if wl.kv_dtype == torch.float8_e4m3fn else OUT_TOL[wl.q_dtype]
    mabs = max_abs_logit(wl, pairs) if wl.q_dtype == torch.float32 else None
    worst = 0.0
    for s, h in pairs:
        L = wl.seq_lens_host[s]
        g = go[s, h].double().numpy()
        if L == 0:
            assert np.all(g == 0.0), f"out[{s},{h}] of an empty sequence is not zero"
            continue
        t = tol if mabs is None else tol + 2.0 ** -21 * mabs[(s, h)]
        worst = max(worst, _tol.check(g, ro[s, h], wl.q_dtype, t, f"out[{s},{h}] L={L}"))
    return worst


# ---- the five workloads at oracle-sized scale, every (seq, head) pair ----------

@pytest.mark.parametrize("name", list(W.SMALL_SPECS))
def test_v1_parity_small(name):
    wl = W.generate(W.SMALL_SPECS[name], poison=True)
    go = run_v1(wl.to(DEV))
    worst = compare(wl, go, run_dense(wl))
    say(f"  {name}: worst {worst:.3g}")


def _sample_pairs(wl, n=10, seed=0):
    rng = np.random.default_rng(seed)
    S, H = wl.num_seqs, wl.num_heads
    pairs = {(0, 0), (S - 1, H - 1)}
    lens = wl.seq_lens_host
    pairs.add((int(np.argmax(lens)), int(rng.integers(H))))
    for s in (i for i, L in enumerate(lens) if L in (0, 1)):
        pairs.add((s, int(rng.integers(H))))
    while len(pairs) < min(n, S * H):
        pairs.add((int(rng.integers(S)), int(rng.integers(H))))
    return sorted(pairs)


@pytest.mark.parametrize("name", ["batched_gqa", "ragged_alibi", "fp8_kv", "long_gqa"])
def test_v1_full_size_sampled(name):
    wl_dev = W.generate(W.SPECS[name], device=DEV, poison=False)
    go = run_v1(wl_dev)
    wl = wl_dev.to("cpu")
    del wl_dev
    torch.cuda.empty_cache()
    assert torch.isfinite(go.float()).all()
    pairs = _sample_pairs(wl)
    worst = compare(wl, go, run_dense(wl, pairs), pairs)
    say(f"  {name}: {len(pairs)} pairs, worst {worst:.3g}")


# ---- edges -------------------------------------------------------------------------

EDGE_LENS = [0, 1, 2, 15, 16, 17, 511, 512, 513, 1000, 1536, 0, 2049]


@pytest.mark.parametrize("q,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                  ("f32", "fp8_e4m3"), ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("D", [64, 80, 96, 112, 120, 128, 192, 256])
def test_v1_edge_dtypes_head_sizes(q, kv, D):
    if kv == "fp8_e4m3" and D % 16:
        pytest.skip("head size not a multiple of 16 fp8 elements")
    ks, vs = (0.05, 0.04) if kv == "fp8_e4m3" else (1.0, 1.0)
    spec = W.Spec(f"v1_edge_{q}_{kv}_{D}", 6, 2, D, 16, q, kv, lambda g: EDGE_LENS,
                  pool=lambda n: n + 9, alibi=(D % 32 == 16 or D == 256), k_scale=ks, v_scale=vs, seed=D)
    wl = W.generate(spec, poison=True)
    compare(wl, run_v1(wl.to(DEV)), run_dense(wl))


@pytest.mark.parametrize("BS", [1, 2, 4, 8, 16, 32, 64, 256, 512])
def test_v1_edge_block_sizes(BS):
    spec = W.Spec(f"v1_bs{BS}", 8, 2, 128, BS, "bf16", "bf16", lambda g: [1, BS - 1, BS, BS + 1, 1300, 0],
                  pool=lambda n: n + 3, alibi=True, seed=BS)
    wl = W.generate(spec, poison=True)
    compare(wl, run_v1(wl.to(DEV)), run_dense(wl))


def test_v1_many_query_heads_per_kv_head():
    """gqa = 40 > 16: three head groups per kv head, the last one partial."""
    spec = W.Spec("v1_gqa40", 80, 2, 128, 16, "f16", "f16", lambda g: [700, 2600, 0, 513],
                  pool=lambda n: n + 5, alibi=True, seed=40)
    wl = W.generate(spec, poison=True)
    compare(wl, run_v1(wl.to(DEV)), run_dense(wl))


def test_v1_all_sequences_empty():
    spec = W.Spec("v1_empty", 8, 2, 64, 16, "bf16", "bf16", lambda g: [0, 0, 0], pool=lambda n: 4, seed=1)
    wl = W.generate(spec, poison=True)
    wl.max_seq_len = 0
    assert torch.all(run_v1(wl.to(DEV)) == 0)


@pytest.mark.parametrize("kv,q,BS", [("bf16", "bf16", 16), ("f32", "f32", 8), ("fp8_e4m3", "f16", 32),
                                     ("f16", "f16", 128)])
def test_v1_block_table_one_hot_probe(kv, q, BS):
    """Sequence s has K = 0 except its token tau = s, where scale * K[tau, 0] =
    200 with q = e_0: every other token's weight, in its own partition or in
    another, underflows to 0 in float32, so the output is V[tau] bit-exactly.
    tau sweeps every token of a 3-partition sequence, one sequence per tau."""
    L = 2 * 512 + 37
    H, KVH, D = 2, 1, 64
    spec = W.Spec("v1_probe", H, KVH, D, BS, q, kv, lambda g: [L] * L, pool=lambda n: n + 7, seed=BS + 1)
    wl = W.generate(spec, poison=True)
    n = (L + BS - 1) // BS
    wl.query.zero_()
    wl.query[:, :, 0] = 1.0
    c = 448.0 if kv == "fp8_e4m3" else 16.0
    wl.scale = 200.0 / c
    t = torch.arange(n * BS)
    vals = (torch.arange(D)[:, None] % 13 + (t[None, :] % 11) * 0.25 - 2.0).to(torch.float32)
    vpat = vals.reshape(D, n, BS).permute(1, 0, 2).unsqueeze(1).to(wl.kv_dtype)
    for s in range(L):
        blocks = wl.block_tables[s, :n].long()
        wl.key_cache[blocks] = 0.0
        wl.value_cache[blocks] = vpat
        b = int(wl.block_tables[s, s // BS])
        wl.key_cache[b, 0, 0, s % BS, 0] = c
    go = run_v1(wl.to(DEV))
    want = vpat.permute(1, 2, 0, 3).reshape(D, n * BS)[:, :L].to(torch.float64).to(wl.q_dtype)
    for s in range(L):
        for h in range(H):
            assert torch.equal(go[s, h], want[:, s]), f"tau={s}: wrong row selected"


def test_v1_matches_v2_and_is_deterministic():
    wl = W.generate(W.SMALL_SPECS["ragged_alibi"], poison=True)
    d = wl.to(DEV)
    a, b = run_v1(d), run_v1(d)
    assert torch.equal(a, b), "V1 is not deterministic"
    v2 = pav2.decode(d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, d.num_kv_heads,
                     d.scale, d.block_size, d.max_seq_len, alibi_slopes=d.alibi_slopes)[0].cpu()
    diff = (a.float() - v2.float()).abs().max().item()
    assert diff <= 4e-3, f"V1 and V2 differ by {diff}"


# ---- dispatch ------------------------------------------------------------------------

@pytest.mark.parametrize("lens,expect_v1", [([300, 511, 1, 0, 512], True), ([5000, 3001], False)])
def test_forward_decode_dispatch(lens, expect_v1):
    spec = W.Spec("dispatch", 16, 4, 128, 16, "bf16", "bf16", lambda g: lens, pool=lambda n: n + 3,
                  alibi=True, seed=len(lens))
    wl = W.generate(spec, poison=True)
    p = pav2.plan(wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_size, wl.block_size,
                  wl.max_num_partitions, pav2.BF16, pav2.BF16)
    assert p["use_v1"] == (1 if expect_v1 else 0)
    d = wl.to(DEV)
    out = pav2.forward_decode(d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens,
                              d.num_kv_heads, d.scale, d.block_size, d.max_seq_len,
                              alibi_slopes=d.alibi_slopes).cpu()
    compare(wl, out, run_dense(wl))


def test_v1_alibi_long_context_frame():
    """ALiBi at 200 partitions plus one token: slopes up to 0.5 put the absolute
    partition maxima near 7e4 (log2 units), where float32 steps are 2^-7, yet
    the output depends on the last two partitions' relative weights.  The
    single pass merges them relative to the sequence's last token."""
    L = 200 * 512 + 1
    spec = W.Spec("v1_alibi_long", 8, 2, 64, 16, "f16", "f16", lambda g: [L, 513], pool=lambda n: n + 3,
                  alibi=True, seed=31)
    wl = W.generate(spec, poison=True)
    worst = compare(wl, run_v1(wl.to(DEV)), run_dense(wl))
    say(f"  worst {worst:.3g}")
