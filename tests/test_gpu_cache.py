"""KV-cache write on the GPU (pav2_reshape_and_cache through the C ABI) against
the oracle, byte for byte.

Both sides start from the same poisoned caches (every byte 0xFF, NaN in all
four formats), so a write to a wrong place shows up as well as a wrong value.
Slot patterns: whole sequences written through their block tables (runs of
consecutive slots, the prefill case), runs starting mid-block, one token per
sequence at its last position (the decode step), a random permutation with
padding (-1) and slots past the pool (which write nothing).
"""
import numpy as np
import pytest
import torch

import oracle
import decode_attention_paged_v2_amd as pav2

pytestmark = pytest.mark.gpu

DEV = "cuda"
_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}
_CODE = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16, "fp8_e4m3": oracle.FP8_E4M3}
PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f32", "fp8_e4m3"), ("f16", "fp8_e4m3"),
         ("bf16", "fp8_e4m3")]


def poisoned(nb, kvh, d, bs, cache_dt):
    es = torch.empty((), dtype=_TD[cache_dt]).element_size()
    x = 16 // es
    kc = torch.full((nb, kvh, d // x, bs, 16), 0xFF, dtype=torch.uint8).view(_TD[cache_dt])
    vc = torch.full((nb, kvh, d, bs * es), 0xFF, dtype=torch.uint8).view(_TD[cache_dt])
    return kc, vc


def slots_for(pattern, T, nb, bs, gen):
    n = nb * bs
    if pattern == "prefill":          # sequences of ragged lengths through shuffled block tables
        lens, pos, out = [1, 15, 16, 17, 100, 513, 7], 0, []
        perm = torch.randperm(nb, generator=gen)
        while len(out) < T:
            L = lens[len(out) % len(lens)]
            nblk = (L + bs - 1) // bs
            if pos + nblk > nb:
                break
            blocks = perm[pos:pos + nblk]
            pos += nblk
            t = torch.arange(L)
            out.extend((blocks[t // bs] * bs + t % bs).tolist())
        out = out[:T]
        return torch.tensor(out + [-1] * (T - len(out)), dtype=torch.int64)
    if pattern == "unaligned":        # consecutive slots from a mid-block start
        return torch.arange(3, 3 + T, dtype=torch.int64) % n
    if pattern == "decode":           # one token per sequence, at a random position of a random block
        return torch.randperm(n, generator=gen)[:T].to(torch.int64)
    if pattern == "padded":           # random distinct slots, some padding, some past the pool
        s = torch.randperm(n, generator=gen)[:T].to(torch.int64)
        idx = torch.randperm(T, generator=gen)
        s[idx[: T // 8]] = -1
        s[idx[T // 8: T // 8 + 3]] = n + torch.arange(3)
        return s
    raise ValueError(pattern)


def run_both(in_dt, cache_dt, T, kvh, d, bs, nb, pattern, k_scale=1.0, v_scale=1.0, seed=0, mag=1.0):
    gen = torch.Generator().manual_seed(seed)
    key = (torch.randn(T, kvh, d, generator=gen) * mag).to(_TD[in_dt])
    value = (torch.randn(T, kvh, d, generator=gen) * mag).to(_TD[in_dt])
    slots = slots_for(pattern, T, nb, bs, gen)
    kc, vc = poisoned(nb, kvh, d, bs, cache_dt)
    # the oracle writes copies; slots past the pool are dropped on its side by hand
    ok = slots < nb * bs
    ref_k, ref_v = oracle.reshape_and_cache(key, value, kc, vc, torch.where(ok, slots, -1), block_size=bs,
                                            cache_dtype=_CODE[cache_dt], k_scale=k_scale, v_scale=v_scale)
    gk, gv = kc.to(DEV), vc.to(DEV)
    pav2.reshape_and_cache(key.to(DEV), value.to(DEV), gk, gv, slots.to(DEV),
                           "fp8_e4m3" if cache_dt == "fp8_e4m3" else "auto", k_scale, v_scale)
    torch.cuda.synchronize()
    return gk.cpu(), gv.cpu(), ref_k, ref_v


def assert_same_bytes(got, ref):
    g = got.contiguous().view(torch.uint8).numpy().ravel()
    r = np.ascontiguousarray(ref).view(np.uint8).ravel()
    assert g.shape == r.shape
    bad = np.flatnonzero(g != r)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:5]}: gpu {g[bad[:5]]} oracle {r[bad[:5]]}"


@pytest.mark.parametrize("in_dt,cache_dt", PAIRS)
@pytest.mark.parametrize("d", [64, 80, 128, 256])
@pytest.mark.parametrize("pattern", ["prefill", "unaligned", "decode", "padded"])
def test_write_matches_oracle(in_dt, cache_dt, d, pattern):
    print(f"case {in_dt}->{cache_dt} d={d} {pattern}", flush=True)
    if cache_dt == "fp8_e4m3" and d % 16:
        pytest.skip("fp8 caches need head_size % 16 == 0")
    scaled = cache_dt == "fp8_e4m3"
    gk, gv, rk, rv = run_both(in_dt, cache_dt, T=203, kvh=3, d=d, bs=16, nb=40, pattern=pattern,
                              k_scale=0.05 if scaled else 1.0, v_scale=0.04 if scaled else 1.0,
                              seed=d, mag=30.0 if scaled else 1.0)
    assert_same_bytes(gk, rk)
    assert_same_bytes(gv, rv)


@pytest.mark.parametrize("in_dt,cache_dt", PAIRS)
@pytest.mark.parametrize("d", [96, 112, 120, 192])
def test_write_other_head_sizes(in_dt, cache_dt, d):
    """The remaining supported head sizes, each through a prefill and a padded slot pattern."""
    print(f"case {in_dt}->{cache_dt} d={d}", flush=True)
    if cache_dt == "fp8_e4m3" and d % 16:
        pytest.skip("fp8 caches need head_size % 16 == 0")
    scaled = cache_dt == "fp8_e4m3"
    for pattern in ("prefill", "padded"):
        gk, gv, rk, rv = run_both(in_dt, cache_dt, T=150, kvh=2, d=d, bs=16, nb=30, pattern=pattern,
                                  k_scale=0.05 if scaled else 1.0, v_scale=0.04 if scaled else 1.0,
                                  seed=d + 1, mag=30.0 if scaled else 1.0)
        assert_same_bytes(gk, rk)
        assert_same_bytes(gv, rv)


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 64, 512])
@pytest.mark.parametrize("in_dt,cache_dt", [("bf16", "bf16"), ("f16", "fp8_e4m3"), ("f32", "f32")])
def test_write_block_sizes(bs, in_dt, cache_dt):
    print(f"case bs={bs} {in_dt}->{cache_dt}", flush=True)
    nb = max(4, 2048 // bs)
    for pattern in ("prefill", "padded"):
        gk, gv, rk, rv = run_both(in_dt, cache_dt, T=300, kvh=2, d=128, bs=bs, nb=nb, pattern=pattern, seed=bs)
        assert_same_bytes(gk, rk)
        assert_same_bytes(gv, rv)


@pytest.mark.parametrize("in_dt,cache_dt", PAIRS)
def test_write_with_scales(in_dt, cache_dt):
    """Non-unit scales on same-dtype caches divide too (the inverse of decode's multiply)."""
    print(f"case scaled {in_dt}->{cache_dt}", flush=True)
    gk, gv, rk, rv = run_both(in_dt, cache_dt, T=97, kvh=2, d=96 if cache_dt != "fp8_e4m3" else 112,
                              bs=16, nb=16, pattern="prefill", k_scale=0.37, v_scale=3.1, seed=5, mag=2.0)
    assert_same_bytes(gk, rk)
    assert_same_bytes(gv, rv)


def test_write_head_size_120_and_192():
    for d, pair in ((120, ("bf16", "bf16")), (192, ("bf16", "fp8_e4m3")), (120, ("f32", "f32"))):
        print(f"case d={d} {pair}", flush=True)
        gk, gv, rk, rv = run_both(*pair, T=50, kvh=2, d=d, bs=16, nb=8, pattern="unaligned", seed=d)
        assert_same_bytes(gk, rk)
        assert_same_bytes(gv, rv)


def test_write_fp8_rounding_edges():
    """Values at e4m3 rounding midpoints, past +-448, subnormals and zeros, through the device converter."""
    codes = torch.arange(0, 0x7E, dtype=torch.uint8)
    lo = codes.view(torch.float8_e4m3fn).double()
    hi = (codes + 1).view(torch.float8_e4m3fn).double()
    vals = torch.cat([(lo + hi) / 2, lo, torch.tensor([448.0, 449.0, 464.0, 500.0, 1e30, 2.0 ** -10,
                                                       3 * 2.0 ** -11, 0.0, -0.0])])
    vals = torch.cat([vals, -vals]).float()
    d, kvh = 128, 1
    T = (vals.numel() + d - 1) // d
    flat = torch.zeros(T * d)
    flat[:vals.numel()] = vals
    key = flat.view(T, kvh, d)
    slots = torch.arange(T, dtype=torch.int64)
    kc, vc = poisoned(4, kvh, d, 16, "fp8_e4m3")
    rk, rv = oracle.reshape_and_cache(key, key, kc, vc, slots, block_size=16, cache_dtype=oracle.FP8_E4M3)
    gk, gv = kc.to(DEV), vc.to(DEV)
    pav2.reshape_and_cache(key.to(DEV), key.to(DEV), gk, gv, slots.to(DEV), "fp8_e4m3")
    torch.cuda.synchronize()
    assert_same_bytes(gk.cpu(), rk)
    assert_same_bytes(gv.cpu(), rv)


def test_write_nan_inputs_stay_nan():
    d, kvh, T = 64, 1, 16
    key = torch.randn(T, kvh, d)
    key[3, 0, 5] = float("nan")
    key[7, 0, 60] = float("nan")
    slots = torch.arange(T, dtype=torch.int64)
    for cache_dt in ("f32", "fp8_e4m3"):
        kc, vc = poisoned(2, kvh, d, 16, cache_dt)
        rk, rv = oracle.reshape_and_cache(key, key, kc, vc, slots, block_size=16, cache_dtype=_CODE[cache_dt],
                                          k_scale=0.5, v_scale=0.5)
        gk, gv = kc.to(DEV), vc.to(DEV)
        pav2.reshape_and_cache(key.to(DEV), key.to(DEV), gk, gv, slots.to(DEV),
                               "fp8_e4m3" if cache_dt == "fp8_e4m3" else "auto", 0.5, 0.5)
        torch.cuda.synchronize()
        ok_ref = oracle.decode(_CODE[cache_dt], np.ascontiguousarray(rk).view(np.uint8))
        ok_gpu = oracle.decode(_CODE[cache_dt], gk.cpu().view(torch.uint8).numpy())
        nan = np.isnan(ok_ref)
        assert np.array_equal(nan, np.isnan(ok_gpu))
        assert np.array_equal(ok_ref[~nan], ok_gpu[~nan])


def test_write_zero_tokens_is_a_no_op():
    kc, vc = poisoned(2, 1, 64, 16, "bf16")
    gk, gv = kc.to(DEV), vc.to(DEV)
    e = torch.empty(0, 1, 64, dtype=torch.bfloat16, device=DEV)
    pav2.reshape_and_cache(e, e, gk, gv, torch.empty(0, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu().view(torch.uint8), kc.view(torch.uint8))


def test_write_then_decode_on_gpu():
    """Tokens written by the cache write are what the decode kernels read:
    decode over the written cache matches the oracle's decode over its own write."""
    gen = torch.Generator().manual_seed(21)
    H, kvh, d, bs = 12, 2, 128, 16
    lens = [1, 600, 1300]
    nb = sum((L + bs - 1) // bs for L in lens) + 2
    perm = torch.randperm(nb, generator=gen)
    mbps = max((L + bs - 1) // bs for L in lens)
    bt = torch.full((len(lens), mbps), -1, dtype=torch.int32)
    pos, slots = 0, []
    for s, L in enumerate(lens):
        n = (L + bs - 1) // bs
        bt[s, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
        t = torch.arange(L)
        slots.append(bt[s, t // bs].long() * bs + t % bs)
    slots = torch.cat(slots)
    T = slots.numel()
    key = torch.randn(T, kvh, d, generator=gen).to(torch.bfloat16)
    value = torch.randn(T, kvh, d, generator=gen).to(torch.bfloat16)
    kc, vc = poisoned(nb, kvh, d, bs, "fp8_e4m3")
    rk, rv = oracle.reshape_and_cache(key, value, kc, vc, slots, block_size=bs, cache_dtype=oracle.FP8_E4M3,
                                      k_scale=0.05, v_scale=0.04)
    gk, gv = kc.to(DEV), vc.to(DEV)
    pav2.reshape_and_cache(key.to(DEV), value.to(DEV), gk, gv, slots.to(DEV), "fp8_e4m3", 0.05, 0.04)
    q = torch.randn(len(lens), H, d, generator=gen).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32)
    out = pav2.decode(q.to(DEV), gk, gv, bt.to(DEV), sl.to(DEV), kvh, d ** -0.5, bs, max(lens),
                      kv_cache_dtype="fp8_e4m3", k_scale=0.05, v_scale=0.04)[0]
    torch.cuda.synchronize()
    kref = torch.from_numpy(np.ascontiguousarray(rk)).view(torch.float8_e4m3fn).reshape(kc.shape)
    vref = torch.from_numpy(np.ascontiguousarray(rv)).view(torch.float8_e4m3fn).reshape(vc.shape)
    r = oracle.paged_attention_v2(q, kref, vref, bt, sl, num_kv_heads=kvh, scale=d ** -0.5, block_size=bs,
                                  max_num_partitions=3, q_dtype=oracle.BF16, kv_dtype=oracle.FP8_E4M3,
                                  k_scale=0.05, v_scale=0.04)
    ref = torch.from_numpy(r["out"]).to(torch.bfloat16).double()
    err = (out.cpu().double() - ref).abs().max().item()
    assert err <= 1e-2, err


@pytest.mark.parametrize("config", ["long_gqa", "fp8_kv"])
def test_write_full_size_sampled(config):
    """The whole context of a full-size workload written in one call, exactly as
    the cache-write benchmark launches it; sampled tokens against the oracle,
    every token against torch's own conversions on the device."""
    from decode_attention_paged_v2_amd import workloads as W
    print(f"case full-size cache write {config}", flush=True)
    sp = W.SPECS[config]
    wl = W.cache_write_workload(sp, DEV)
    torch.cuda.synchronize()
    kvdt = "fp8_e4m3" if wl.cache_dtype == torch.float8_e4m3fn else "auto"
    pav2.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, wl.slot_mapping, kvdt,
                           wl.k_scale, wl.v_scale)
    torch.cuda.synchronize()
    T, kvh, d = wl.key.shape
    bs = wl.value_cache.shape[3]
    x = wl.key_cache.shape[4]
    blk, off = wl.slot_mapping // bs, wl.slot_mapping % bs
    # every token, on the device: the cache rows gathered back with torch indexing
    kg = wl.key_cache[blk, :, :, off, :].reshape(T, kvh, d)
    vg = wl.value_cache[blk, :, :, off]
    if kvdt == "auto":
        assert torch.equal(kg, wl.key) and torch.equal(vg, wl.value)
    else:
        def q(t, s):
            return (t.float() / torch.tensor(s, dtype=torch.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
        for i in range(0, T, 1 << 16):      # chunks keep the float32 temporaries small
            sl = slice(i, i + (1 << 16))
            assert torch.equal(kg[sl].view(torch.uint8), q(wl.key[sl], wl.k_scale).view(torch.uint8))
            assert torch.equal(vg[sl].view(torch.uint8), q(wl.value[sl], wl.v_scale).view(torch.uint8))
    # sampled tokens against the oracle: written into a small cache at slots 0..n-1
    gen = torch.Generator().manual_seed(3)
    idx = torch.cat([torch.tensor([0, T - 1]), torch.randint(0, T, (1022,), generator=gen)])
    n = idx.numel()
    kc, vc = poisoned((n + bs - 1) // bs, kvh, d, bs, "fp8_e4m3" if kvdt != "auto" else
                      {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[wl.key.dtype])
    rk, rv = oracle.reshape_and_cache(wl.key[idx.to(DEV)].cpu(), wl.value[idx.to(DEV)].cpu(), kc, vc,
                                      torch.arange(n), block_size=bs, cache_dtype=_CODE[
                                          "fp8_e4m3" if kvdt != "auto" else
                                          {torch.bfloat16: "bf16", torch.float16: "f16",
                                           torch.float32: "f32"}[wl.key.dtype]],
                                      k_scale=wl.k_scale, v_scale=wl.v_scale)
    rk = torch.from_numpy(np.ascontiguousarray(rk)).view(torch.uint8).reshape(kc.shape[0], kvh, d // x, bs, -1)
    rv = torch.from_numpy(np.ascontiguousarray(rv)).view(torch.uint8).reshape(vc.shape[0], kvh, d, -1)
    es = wl.key_cache.element_size()
    j = torch.arange(n)
    want_k = rk.view(wl.key_cache.dtype)[j // bs, :, :, j % bs, :].reshape(n, kvh, d)
    want_v = rv.view(wl.value_cache.dtype)[j // bs, :, :, j % bs]
    ii = idx.to(DEV)
    assert torch.equal(kg[ii].cpu().view(torch.uint8), want_k.view(torch.uint8)), es
    assert torch.equal(vg[ii].cpu().view(torch.uint8), want_v.view(torch.uint8))


@pytest.mark.parametrize("cache_dt", ["fp8_e4m3", "bf16", "f16"])
@pytest.mark.parametrize("scale", [0.05, 0.04, 0.37, 3.1, 2.0 ** -90, 2.0 ** 90])
def test_write_scaled_quotients_at_rounding_edges(cache_dt, scale):
    """Inputs whose quotient by the scale lies within a float32 ulp of a rounding
    midpoint of the cache dtype (and of representable values), plus inputs
    around the magnitudes where the kernel switches between its FMA-corrected
    quotient and the division itself: every byte must match the oracle's IEEE
    float32 division followed by round-to-nearest-even."""
    print(f"case quotient edges {cache_dt} scale={scale}", flush=True)
    gen = torch.Generator().manual_seed(31)
    if cache_dt == "fp8_e4m3":
        codes = torch.arange(0, 0x7E, dtype=torch.uint8)
        lo = codes.view(torch.float8_e4m3fn).double()
        hi = (codes + 1).view(torch.float8_e4m3fn).double()
    else:
        dt = _TD[cache_dt]
        codes = torch.randint(0, 0x7B00 if cache_dt == "f16" else 0x7F00, (4000,), generator=gen, dtype=torch.int32)
        lo = codes.to(torch.int16).view(dt).double()
        hi = (codes + 1).to(torch.int16).view(dt).double()
    targets = torch.cat([(lo + hi) / 2, lo])
    x = (targets * scale).float()                               # RN32(target * s)
    up = torch.nextafter(x, torch.full_like(x, float("inf")))
    dn = torch.nextafter(x, torch.full_like(x, float("-inf")))
    special = torch.tensor([2.0 ** -97, 2.0 ** -96, 2.0 ** -95, 1.5 * 2.0 ** -96, 2.0 ** -126, 1e-40, 0.0,
                            2.0 ** 99, 2.0 ** 100, 2.0 ** 101, 3e38], dtype=torch.float64)
    vals = torch.cat([x, up, dn, special.float(), (special * scale).float()])
    vals = torch.cat([vals, -vals])
    vals = vals[torch.isfinite(vals)]
    d, kvh = 128, 1
    T = (vals.numel() + d - 1) // d
    flat = torch.zeros(T * d)
    flat[:vals.numel()] = vals
    key = flat.view(T, kvh, d)
    value = key.flip(0).contiguous()
    slots = torch.arange(T, dtype=torch.int64)
    nb = (T + 15) // 16
    kc, vc = poisoned(nb, kvh, d, 16, cache_dt)
    gk, gv = kc.to(DEV), vc.to(DEV)
    # fp8 caches take the float32 values; a 16-bit cache takes inputs of its
    # own dtype (the values rounded to it)
    if cache_dt != "fp8_e4m3":
        key, value = key.to(_TD[cache_dt]), value.to(_TD[cache_dt])
    rk, rv = oracle.reshape_and_cache(key, value, kc, vc, slots, block_size=16, cache_dtype=_CODE[cache_dt],
                                      k_scale=scale, v_scale=scale)
    pav2.reshape_and_cache(key.to(DEV), value.to(DEV), gk, gv, slots.to(DEV),
                           "fp8_e4m3" if cache_dt == "fp8_e4m3" else "auto", scale, scale)
    torch.cuda.synchronize()
    assert_same_bytes(gk.cpu(), rk)
    assert_same_bytes(gv.cpu(), rv)
