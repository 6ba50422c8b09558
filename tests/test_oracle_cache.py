"""Pins for the oracle's KV-cache write (CPU only).

The write is the inverse of the decode gather (page "paged_attn.py",
write_to_paged_cache / split_kv_cache): a token's key and value go to slot
`slot_mapping[t]` of the paged layouts, divided by k_scale / v_scale and
rounded to the cache dtype.  Each test checks the oracle against something
other than itself: numpy's and torch's own float conversions, torch views of
the cache (not index arithmetic), closed forms for rounding ties and
saturation, and torch's scaled_dot_product_attention after a write.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_v2_amd import workloads as W
from _brute import f32

_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
       "fp8_e4m3": torch.float8_e4m3fn}
_CODE = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16, "fp8_e4m3": oracle.FP8_E4M3}


def _random_f32(n, seed):
    """float32 values over the whole range: random bit patterns plus N(0,1)-scaled values."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    normal = (rng.standard_normal(n) * rng.choice([1e-6, 1e-3, 1.0, 30.0, 1e3, 1e5], n)).astype(np.float32)
    return np.concatenate([vals, normal])


# ---- encoders against library conversions ------------------------------------

def test_encode_f16_matches_numpy():
    x = _random_f32(200_000, 1)
    got = oracle.encode(oracle.F16, x).view(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_encode_bf16_matches_torch():
    x = _random_f32(200_000, 2)
    got = oracle.encode(oracle.BF16, x).view(np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_encode_e4m3_matches_torch_in_range():
    x = _random_f32(200_000, 3)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    got = oracle.encode(oracle.FP8_E4M3, x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_encode_e4m3_saturates_and_keeps_nan():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf], dtype=np.float32)
    got = oracle.encode(oracle.FP8_E4M3, x)
    assert list(got) == [0x7E] * 6 + [0xFE] * 2
    got = oracle.encode(oracle.FP8_E4M3, np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(np.isnan(oracle.decode(oracle.FP8_E4M3, got)))


def test_encode_e4m3_all_codes_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(oracle.FP8_E4M3, codes)
    ok = ~np.isnan(vals)
    got = oracle.encode(oracle.FP8_E4M3, vals[ok].astype(np.float32))
    assert np.array_equal(got, codes[ok])


def test_encode_e4m3_ties_to_even():
    # midpoints between neighbouring codes c, c+1 (same sign, finite) round to the even code
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo = oracle.decode(oracle.FP8_E4M3, codes)
    hi = oracle.decode(oracle.FP8_E4M3, codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)     # midpoints are exact in float32
    got = oracle.encode(oracle.FP8_E4M3, mid)
    want = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.encode(oracle.FP8_E4M3, -mid), want | 0x80)


# ---- the write itself ----------------------------------------------------------

def _caches(nb, kvh, d, bs, cache_dt, gen):
    """Poisoned caches: every byte 0xFF (NaN in all four formats)."""
    es = W.elem_size(_TD[cache_dt])
    x = 16 // es
    kc = torch.full((nb, kvh, d // x, bs, 16), 0xFF, dtype=torch.uint8).view(_TD[cache_dt])
    vc = torch.full((nb, kvh, d, bs * es), 0xFF, dtype=torch.uint8).view(_TD[cache_dt])
    return kc, vc


def _slots(T, nb, bs, gen, pad=0):
    s = torch.randperm(nb * bs, generator=gen)[:T].to(torch.int64)
    if pad:
        s[torch.randperm(T, generator=gen)[:pad]] = -1
    return s


def _as(t_bytes, like):
    return torch.from_numpy(np.ascontiguousarray(t_bytes)).view(like.dtype).reshape(like.shape)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bs,d", [(8, 64), (16, 80), (32, 128)])
def test_write_round_trip_via_views(dt, bs, d):
    """Same-dtype write with unit scales stores the input bits at the slot (torch views)."""
    gen = torch.Generator().manual_seed(11)
    T, kvh, nb = 37, 3, 9
    key = torch.randn(T, kvh, d, generator=gen).to(_TD[dt])
    value = torch.randn(T, kvh, d, generator=gen).to(_TD[dt])
    kc, vc = _caches(nb, kvh, d, bs, dt, gen)
    slots = _slots(T, nb, bs, gen, pad=4)
    kb, vb = oracle.reshape_and_cache(key, value, kc, vc, slots, block_size=bs, cache_dtype=_CODE[dt])
    kw, vw = _as(kb, kc), _as(vb, vc)
    x = kc.shape[-1]
    written = set()
    for t in range(T):
        sl = int(slots[t])
        if sl < 0:
            continue
        b, o = divmod(sl, bs)
        written.add(sl)
        # key_cache[b, g, :, o, :] flattened over (d/x, x) is the head-dim row
        krow = kw[b, :, :, o, :].reshape(kvh, d)
        vrow = vw[b, :, :, o]
        assert torch.equal(krow.view(torch.uint8) if dt == "fp8_e4m3" else krow, key[t])
        assert torch.equal(vrow, value[t])
    # every slot not written keeps its poison bytes
    kflat = kw.view(torch.uint8).reshape(nb, kvh, d // x, bs, -1).permute(0, 3, 1, 2, 4).reshape(nb * bs, -1)
    vflat = vw.view(torch.uint8).reshape(nb, kvh, d, bs, -1).permute(0, 3, 1, 2, 4).reshape(nb * bs, -1)
    untouched = torch.tensor([s not in written for s in range(nb * bs)])
    assert torch.all(kflat[untouched] == 0xFF) and torch.all(vflat[untouched] == 0xFF)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_write_fp8_scaled_matches_library(dt):
    """fp8 write = torch's e4m3 cast of clamp(float32(x) / float32(scale), +-448)."""
    gen = torch.Generator().manual_seed(12)
    T, kvh, d, bs, nb = 50, 2, 128, 32, 4
    key = (torch.randn(T, kvh, d, generator=gen) * 30).to(_TD[dt])
    value = (torch.randn(T, kvh, d, generator=gen) * 30).to(_TD[dt])
    kc, vc = _caches(nb, kvh, d, bs, "fp8_e4m3", gen)
    slots = _slots(T, nb, bs, gen)
    ks, vs = 0.05, 0.04
    kb, vb = oracle.reshape_and_cache(key, value, kc, vc, slots, block_size=bs,
                                      cache_dtype=oracle.FP8_E4M3, k_scale=ks, v_scale=vs)
    kw, vw = _as(kb, kc), _as(vb, vc)

    def q(t, sc):
        a = t.float().numpy() / np.float32(f32(sc))       # IEEE float32 division
        a = np.clip(a, -448.0, 448.0)
        return torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8)
    kq, vq = q(key, ks), q(value, vs)
    for t in range(T):
        b, o = divmod(int(slots[t]), bs)
        assert torch.equal(kw[b, :, :, o, :].reshape(kvh, d).view(torch.uint8), kq[t])
        assert torch.equal(vw[b, :, :, o].view(torch.uint8), vq[t])


def test_write_then_decode_matches_dense_attention():
    """Sequences written token by token through slot_mapping decode to softmax(qK^T)V of the inputs."""
    gen = torch.Generator().manual_seed(13)
    H, kvh, d, bs = 8, 2, 64, 16
    lens = [1, 17, 700]
    nb = sum((L + bs - 1) // bs for L in lens) + 3
    perm = torch.randperm(nb, generator=gen)
    mbps = max((L + bs - 1) // bs for L in lens)
    bt = torch.full((len(lens), mbps), -1, dtype=torch.int32)
    pos = 0
    keys, values, slots = [], [], []
    for s, L in enumerate(lens):
        n = (L + bs - 1) // bs
        bt[s, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
        k = torch.randn(L, kvh, d, generator=gen).to(torch.bfloat16)
        v = torch.randn(L, kvh, d, generator=gen).to(torch.bfloat16)
        keys.append(k)
        values.append(v)
        t = torch.arange(L)
        slots.append(bt[s, t // bs].long() * bs + t % bs)
    kc, vc = _caches(nb, kvh, d, bs, "bf16", gen)
    kb, vb = oracle.reshape_and_cache(torch.cat(keys), torch.cat(values), kc, vc, torch.cat(slots),
                                      block_size=bs, cache_dtype=oracle.BF16)
    kw, vw = _as(kb, kc), _as(vb, vc)
    q = torch.randn(len(lens), H, d, generator=gen).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32)
    r = oracle.paged_attention_v2(q, kw, vw, bt, sl, num_kv_heads=kvh, scale=d ** -0.5, block_size=bs,
                                  max_num_partitions=2, q_dtype=oracle.BF16, kv_dtype=oracle.BF16)
    gqa = H // kvh
    for s, L in enumerate(lens):
        k = keys[s].double().permute(1, 0, 2).repeat_interleave(gqa, 0)
        v = values[s].double().permute(1, 0, 2).repeat_interleave(gqa, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[s].double()[None, :, None, :], k[None], v[None], scale=f32(d ** -0.5))[0, :, 0, :]
        assert np.max(np.abs(r["out"][s] - ref.numpy())) < 1e-12


def test_write_rejects_bad_arguments():
    gen = torch.Generator().manual_seed(14)
    key = torch.randn(4, 1, 64, generator=gen)
    kc, vc = _caches(2, 1, 64, 16, "f32", gen)
    with pytest.raises(ValueError):      # slot past the pool
        oracle.reshape_and_cache(key, key, kc, vc, torch.tensor([0, 1, 2, 32]), block_size=16,
                                 cache_dtype=oracle.F32)
    with pytest.raises(ValueError):      # cache dtype neither the input's nor fp8
        oracle.reshape_and_cache(key, key, kc, vc, torch.tensor([0, 1, 2, 3]), block_size=16,
                                 cache_dtype=oracle.BF16)
