"""The allocation-free V2 entry point (pav2_paged_attention_v2_noalloc, through
the C ABI) against the V2 entry point with caller buffers, on consecutive
calls that share the library's per-device scratch: the second call is
smaller than the first, so everything a stale read could see is the first
call's data.  The two entry points run the same kernels, so their outputs
must agree bit for bit; each output is also held to the oracle's tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import _tol
import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 2e-3}

FIRST = W.SMALL_SPECS["ragged_alibi"]     # 16 ragged sequences up to 4096 tokens, ALiBi, f16, d 80
SECOND = W.Spec("noalloc_second", 32, 8, 80, 16, "f16", "f16", lambda g: [700, 3, 1300],
                pool=lambda n: n + 5, alibi=True, seed=77)
THIRD = W.SMALL_SPECS["fp8_kv"]            # another dtype pair and layout after both


def _args(d):
    return ((d.query, d.key_cache, d.value_cache, d.num_kv_heads, d.scale, d.block_tables, d.seq_lens,
             d.block_size, d.max_seq_len),
            dict(alibi_slopes=d.alibi_slopes, k_scale=d.k_scale, v_scale=d.v_scale,
                 kv_cache_dtype="fp8_e4m3" if d.kv_dtype == torch.float8_e4m3fn else "auto"))


def _one(spec):
    print(f"case noalloc {spec.name}", flush=True)
    wl = W.generate(spec, poison=True)
    d = wl.to(DEV)
    a, kw = _args(d)
    got = torch.full_like(d.query, float("nan"))
    pav2.paged_attention_v2_noalloc(got, *a, **kw)
    ref_out = pav2.decode(d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, d.num_kv_heads,
                          d.scale, d.block_size, d.max_seq_len, **kw)[0]   # caller-allocated workspace
    torch.cuda.synchronize()
    g, r = got.cpu(), ref_out.cpu()
    assert torch.equal(g.view(torch.int16 if g.element_size() == 2 else torch.int32),
                       r.view(torch.int16 if r.element_size() == 2 else torch.int32)), \
        "noalloc output differs from the V2 entry point's"
    o = oracle.paged_attention_v2(wl.query, wl.key_cache, wl.value_cache, wl.block_tables, wl.seq_lens,
                                  num_kv_heads=wl.num_kv_heads, scale=wl.scale, block_size=wl.block_size,
                                  max_num_partitions=wl.max_num_partitions, q_dtype=oracle.dtype_code(wl.q_dtype),
                                  kv_dtype=oracle.dtype_code(wl.kv_dtype), alibi_slopes=wl.alibi_slopes,
                                  k_scale=wl.k_scale, v_scale=wl.v_scale)
    tol = 1e-2 if wl.kv_dtype == torch.float8_e4m3fn else TOL[wl.q_dtype]
    for s in range(wl.num_seqs):
        L = wl.seq_lens_host[s]
        P = (L + 511) // 512
        for h in range(wl.num_heads):
            extra = 0.0
            if P:
                extra = _tol.tmp_rounding_budget(o["max_logits"][s, h, :P], o["exp_sums"][s, h, :P],
                                                 o["tmp_output"][s, h, :P], wl.q_dtype)
            _tol.check(g[s, h].double().numpy(), o["out"][s, h], wl.q_dtype, tol, f"out[{s},{h}] L={L}", extra)


def test_noalloc_matches_v2_on_consecutive_calls():
    assert pav2.noalloc_scratch_bytes() == 64 << 20
    _one(FIRST)
    _one(SECOND)    # smaller: the scratch still holds the first call's partitions
    _one(THIRD)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # 256 seqs x 32 heads x 64 partitions x (80 * 2 + 8) bytes = 88 MB > 64 MiB:
    # rejected before any launch (the device tensors are never touched)
    q = torch.zeros((256, 32, 80), dtype=torch.float16, device=DEV)
    kc = torch.zeros((1, 8, 10, 16, 8), dtype=torch.float16, device=DEV)
    vc = torch.zeros((1, 8, 80, 16), dtype=torch.float16, device=DEV)
    bt = torch.zeros((256, 2048), dtype=torch.int32, device=DEV)
    sl = torch.zeros((256,), dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(pav2.Pav2Error) as e:
        pav2.paged_attention_v2_noalloc(out, q, kc, vc, 8, 0.1, bt, sl, 16, 32768)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
