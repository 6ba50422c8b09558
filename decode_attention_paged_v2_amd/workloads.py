"""Seeded synthetic inputs for PagedAttention V2 decode.

This module only draws random inputs and lays them out in the paged cache
format; it holds none of the attention arithmetic, and both the HIP path and
the float64 oracle are fed from it.

Layouts (page "paged_attn.py", split_kv_cache and the shape comments of
_forward_decode_pytorch):

* query        [num_seqs, num_heads, head_size]
* key_cache    [num_blocks, num_kv_heads, head_size // x, block_size, x]
               with x = 16 // element_size (16-byte vectors)
* value_cache  [num_blocks, num_kv_heads, head_size, block_size]
* block_tables [num_seqs, max_blocks_per_seq] int32, logical -> physical
* seq_lens     [num_seqs] int32

Recipe (one torch.Generator per workload, seeded; draw order seq_lens ->
block permutation -> query -> key cache -> value cache):

* values are N(0, 1) drawn in float32 and cast with round-to-nearest-even;
  fp8 e4m3 caches store clamp(N(0,1) / scale, +-448) so that the dequantised
  value scale * code is N(0,1)-like;
* block tables are consecutive slices of one random permutation of the block
  pool, so blocks are disjoint and shuffled; entries past a sequence's last
  block are -1;
* with ``poison=True`` (correctness runs) every cache slot that no sequence
  references -- unreferenced blocks and slots past seq_len in a sequence's
  last block -- holds NaN, so any read of it shows up in the result.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

PARTITION_SIZE = 512

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
       "fp8_e4m3": torch.float8_e4m3fn}


def elem_size(dtype: torch.dtype) -> int:
    return torch.empty((), dtype=dtype).element_size()


def x_pack(kv_dtype: torch.dtype) -> int:
    """Key-cache packing factor: elements per 16-byte vector."""
    return 16 // elem_size(kv_dtype)


@dataclass
class Workload:
    name: str
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    alibi_slopes: Optional[torch.Tensor]
    num_kv_heads: int
    scale: float
    block_size: int
    max_seq_len: int
    max_num_partitions: int
    k_scale: float = 1.0
    v_scale: float = 1.0
    seq_lens_host: list = field(default_factory=list)

    @property
    def num_seqs(self):
        return self.query.shape[0]

    @property
    def num_heads(self):
        return self.query.shape[1]

    @property
    def head_size(self):
        return self.query.shape[2]

    @property
    def q_dtype(self):
        return self.query.dtype

    @property
    def kv_dtype(self):
        return self.key_cache.dtype

    @property
    def num_blocks(self):
        return self.key_cache.shape[0]

    def to(self, device) -> "Workload":
        mv = lambda t: None if t is None else t.to(device)
        return Workload(self.name, mv(self.query), mv(self.key_cache), mv(self.value_cache),
                        mv(self.block_tables), mv(self.seq_lens), mv(self.alibi_slopes),
                        self.num_kv_heads, self.scale, self.block_size, self.max_seq_len,
                        self.max_num_partitions, self.k_scale, self.v_scale,
                        list(self.seq_lens_host))

    def kv_bytes(self) -> int:
        """Bytes of K and V that one decode step must read: sum_s L_s * kv_h * 2 * d * b."""
        b = elem_size(self.kv_dtype)
        return sum(self.seq_lens_host) * self.num_kv_heads * 2 * self.head_size * b

    def tokens_heads(self) -> int:
        return sum(self.seq_lens_host) * self.num_heads


@dataclass
class Spec:
    """A workload recipe; ``lens`` is a callable (generator) -> list[int]."""
    name: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    lens: object
    pool: object = None          # callable(total_blocks_needed) -> pool size, or None
    alibi: bool = False
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0


def _fill_normal(t: torch.Tensor, g: torch.Generator, quant_scale: float, chunk_rows: int = 256):
    """Fill t (first dim chunked) with N(0,1) values cast to t's dtype."""
    n = t.shape[0]
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        v = torch.randn((r1 - r0,) + tuple(t.shape[1:]), generator=g, dtype=torch.float32,
                        device=t.device)
        if t.dtype == torch.float8_e4m3fn:
            v = (v / quant_scale).clamp_(-448.0, 448.0)
        t[r0:r1] = v.to(t.dtype)


def generate(spec: Spec, device="cpu", poison: bool = False, seed: Optional[int] = None) -> Workload:
    seed = spec.seed if seed is None else seed
    gen_dev = torch.device(device)
    g = torch.Generator(device=gen_dev)
    g.manual_seed(seed)
    gl = torch.Generator()                 # host generator for the integer draws
    gl.manual_seed(seed)

    lens = [int(v) for v in spec.lens(gl)]
    S = len(lens)
    H, KVH, D, BS = spec.num_heads, spec.num_kv_heads, spec.head_size, spec.block_size
    qdt, kvdt = _DT[spec.q_dtype], _DT[spec.kv_dtype]
    x = x_pack(kvdt)
    if D % x:
        raise ValueError("head_size must be a multiple of the key packing factor")

    need = [(L + BS - 1) // BS for L in lens]
    total = sum(need)
    pool = spec.pool(total) if spec.pool else total
    if pool < total:
        raise ValueError("block pool smaller than the blocks the sequences need")
    perm = torch.randperm(pool, generator=gl)
    max_len = max(lens) if lens else 0
    mbps = max(1, max((need or [1])))
    bt = torch.full((S, mbps), -1, dtype=torch.int32)
    off = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[off:off + n].to(torch.int32)
        off += n

    query = torch.randn((S, H, D), generator=g, dtype=torch.float32, device=gen_dev).to(qdt)
    key_cache = torch.empty((pool, KVH, D // x, BS, x), dtype=kvdt, device=gen_dev)
    value_cache = torch.empty((pool, KVH, D, BS), dtype=kvdt, device=gen_dev)
    rows = max(1, (64 << 20) // max(1, KVH * D * BS * 4))
    _fill_normal(key_cache, g, spec.k_scale, rows)
    _fill_normal(value_cache, g, spec.v_scale, rows)

    if poison:
        nan = torch.tensor(float("nan")).to(kvdt).to(gen_dev)
        used = torch.zeros(pool, dtype=torch.bool)
        for s, n in enumerate(need):
            used[bt[s, :n].long()] = True
        unused = (~used).nonzero().flatten().to(gen_dev)
        if unused.numel():
            key_cache[unused] = nan
            value_cache[unused] = nan
        for s, L in enumerate(lens):
            if L % BS:
                last = int(bt[s, need[s] - 1])
                key_cache[last, :, :, L % BS:, :] = nan
                value_cache[last, :, :, L % BS:] = nan

    alibi = None
    if spec.alibi:
        # slope_i = 2^(-8 i / H), i = 1..H (the usual geometric ALiBi slopes)
        alibi = torch.tensor([2.0 ** (-8.0 * (i + 1) / H) for i in range(H)], dtype=torch.float32)

    maxP = max(1, (max_len + PARTITION_SIZE - 1) // PARTITION_SIZE)
    wl = Workload(
        name=spec.name, query=query, key_cache=key_cache, value_cache=value_cache,
        block_tables=bt.to(gen_dev), seq_lens=torch.tensor(lens, dtype=torch.int32).to(gen_dev),
        alibi_slopes=None if alibi is None else alibi.to(gen_dev),
        num_kv_heads=KVH, scale=1.0 / math.sqrt(D), block_size=BS,
        max_seq_len=max_len, max_num_partitions=maxP,
        k_scale=spec.k_scale, v_scale=spec.v_scale, seq_lens_host=lens)
    return wl


# ---- the five workloads at their full sizes ------------------------------

def _fixed(n, L):
    return lambda g: [L] * n


def _uniform(n, lo, hi):
    return lambda g: torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def _log_uniform(n, lo, hi, zeros):
    def f(g):
        u = torch.rand(n, generator=g, dtype=torch.float64)
        lens = torch.floor(torch.exp(u * math.log(hi + 1))).clamp_(lo, hi).long()
        z = torch.randperm(n, generator=g)[:zeros]
        lens[z] = 0
        return lens.tolist()
    return f


SPECS = {
    # 1 seq of 1000 tokens (2 partitions), H = kv_h = 4, d = 64, fp32;
    # 63 blocks taken from a 128-block pool
    "tiny": Spec("tiny", 4, 4, 64, 16, "f32", "f32", _fixed(1, 1000),
                 pool=lambda n: 128, seed=1001),
    # 32 seqs, L ~ U[512, 4096], H = 32, kv_h = 8, d = 128, fp16, 16384-block pool
    "batched_gqa": Spec("batched_gqa", 32, 8, 128, 16, "f16", "f16", _uniform(32, 512, 4096),
                        pool=lambda n: 16384, seed=1002),
    # 4 seqs x 100000 tokens (196 partitions), H = 24, kv_h = 4, d = 256, bf16
    "long_gqa": Spec("long_gqa", 24, 4, 256, 16, "bf16", "bf16", _fixed(4, 100000), seed=1003),
    # 256 seqs, L log-uniform in [1, 32768], 4 of them 0, H = 32, kv_h = 8, d = 80, ALiBi
    "ragged_alibi": Spec("ragged_alibi", 32, 8, 80, 16, "f16", "f16",
                         _log_uniform(256, 1, 32768, 4), alibi=True, seed=1004),
    # 64 seqs x 16384, H = 64, kv_h = 8, d = 128, block 32, e4m3 KV, bf16 q/out
    "fp8_kv": Spec("fp8_kv", 64, 8, 128, 32, "bf16", "fp8_e4m3", _fixed(64, 16384),
                   pool=lambda n: 32768, k_scale=0.05, v_scale=0.04, seed=1005),
}

# Reduced copies with the same head layout, dtypes and length structure, small
# enough for the oracle to finish every (seq, head) pair in seconds while still
# spanning several 16-token tiles, several partitions and ragged tails.
SMALL_SPECS = {
    "tiny": SPECS["tiny"],
    "batched_gqa": Spec("batched_gqa_small", 32, 8, 128, 16, "f16", "f16",
                        lambda g: [512, 4096, 1537, 2000, 777, 3333], pool=lambda n: n + 37,
                        seed=2002),
    "long_gqa": Spec("long_gqa_small", 24, 4, 256, 16, "bf16", "bf16",
                     lambda g: [5000, 3001], pool=lambda n: n + 11, seed=2003),
    "ragged_alibi": Spec("ragged_alibi_small", 32, 8, 80, 16, "f16", "f16",
                         lambda g: [0, 1, 2, 15, 16, 17, 511, 512, 513, 1000, 0, 1025, 2047, 2500,
                                    31, 4096], pool=lambda n: n + 23, alibi=True, seed=2004),
    "fp8_kv": Spec("fp8_kv_small", 64, 8, 128, 32, "bf16", "fp8_e4m3",
                   lambda g: [2048, 1500, 33, 4096], pool=lambda n: n + 19,
                   k_scale=0.05, v_scale=0.04, seed=2005),
}


# ---- KV-cache write inputs ---------------------------------------------------

@dataclass
class CacheWriteWorkload:
    """New tokens to write into a paged cache: key, value [T, kv_h, d] in the
    workload's query dtype, slot_mapping [T] int64, and the (unwritten) caches."""
    name: str
    key: torch.Tensor
    value: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    slot_mapping: torch.Tensor
    k_scale: float
    v_scale: float
    cache_dtype: torch.dtype

    def bytes_moved(self) -> int:
        """Input bytes read plus cache bytes written (key and value)."""
        T, kvh, d = self.key.shape
        return T * kvh * d * 2 * (self.key.element_size() + self.key_cache.element_size())


def cache_write_workload(spec: Spec, device="cpu", decode_step: bool = False,
                         seed: Optional[int] = None) -> CacheWriteWorkload:
    """The whole context of a workload as one write (the prefill of every
    sequence: each sequence's tokens in order, through its shuffled block
    table), or with ``decode_step`` one new token per sequence at position
    seq_len - 1.  Values N(0,1) in the query dtype; the caches are allocated
    empty (their prior contents are not part of the write)."""
    seed = spec.seed if seed is None else seed
    gen_dev = torch.device(device)
    g = torch.Generator(device=gen_dev)
    g.manual_seed(seed + 500)
    gl = torch.Generator()
    gl.manual_seed(seed)
    lens = [int(v) for v in spec.lens(gl)]
    KVH, D, BS = spec.num_kv_heads, spec.head_size, spec.block_size
    in_dt, cdt = _DT[spec.q_dtype], _DT[spec.kv_dtype]
    x = x_pack(cdt)
    need = [(L + BS - 1) // BS for L in lens]
    total = sum(need)
    pool = spec.pool(total) if spec.pool else total
    perm = torch.randperm(pool, generator=gl)
    slots, off = [], 0
    for L, n in zip(lens, need):
        blocks = perm[off:off + n]
        off += n
        t = torch.arange(L - 1, L) if decode_step else torch.arange(L)
        if L > 0:
            slots.append(blocks[t // BS].long() * BS + t % BS)
    slot_mapping = (torch.cat(slots) if slots else torch.empty(0, dtype=torch.int64)).to(gen_dev)
    T = slot_mapping.numel()
    key = torch.randn((T, KVH, D), generator=g, dtype=torch.float32, device=gen_dev).to(in_dt)
    value = torch.randn((T, KVH, D), generator=g, dtype=torch.float32, device=gen_dev).to(in_dt)
    key_cache = torch.empty((pool, KVH, D // x, BS, x), dtype=cdt, device=gen_dev)
    value_cache = torch.empty((pool, KVH, D, BS), dtype=cdt, device=gen_dev)
    return CacheWriteWorkload(spec.name + ("_decode_step" if decode_step else "_prefill"), key, value,
                              key_cache, value_cache, slot_mapping, spec.k_scale, spec.v_scale, cdt)


# ---- paged prefix attention (chunked prefill) inputs -------------------------

@dataclass
class PrefixWorkload:
    """Chunks of new query tokens over sequences whose first context_lens[i]
    tokens are already in the paged cache.  query [T, H, d], key / value
    [T, kv_h, d] (the chunks' own keys and values), block tables covering
    context + chunk, and slot_mapping [T] (int64): where each chunk token's
    key / value go in the cache.  Chunk slots in the cache hold NaN until
    written."""
    query: torch.Tensor
    key: torch.Tensor
    value: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor
    query_start_loc: torch.Tensor
    context_lens: torch.Tensor
    slot_mapping: torch.Tensor
    num_kv_heads: int
    block_size: int
    ctx_host: list
    qlen_host: list

    @property
    def max_query_len(self):
        return max(self.qlen_host) if self.qlen_host else 0

    def to(self, device) -> "PrefixWorkload":
        mv = lambda t: t.to(device)
        return PrefixWorkload(mv(self.query), mv(self.key), mv(self.value), mv(self.key_cache),
                              mv(self.value_cache), mv(self.block_tables), mv(self.query_start_loc),
                              mv(self.context_lens), mv(self.slot_mapping), self.num_kv_heads,
                              self.block_size, list(self.ctx_host), list(self.qlen_host))


def prefix_workload(ctx_lens, q_lens, num_heads, num_kv_heads, head_size, block_size, dtype="bf16",
                    seed=0, device="cpu", extra_blocks=3) -> PrefixWorkload:
    """Seeded inputs: N(0,1) values in `dtype`, shuffled disjoint block tables."""
    dt = _DT[dtype]
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    gl = torch.Generator()
    gl.manual_seed(seed)
    S, H, KVH, D, BS = len(ctx_lens), num_heads, num_kv_heads, head_size, block_size
    x = x_pack(dt)
    need = [(c + q + BS - 1) // BS for c, q in zip(ctx_lens, q_lens)]
    pool = sum(need) + extra_blocks
    perm = torch.randperm(pool, generator=gl)
    bt = torch.full((S, max(1, max(need or [1]))), -1, dtype=torch.int32)
    off, slots = 0, []
    for s, n in enumerate(need):
        bt[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
        t = torch.arange(ctx_lens[s], ctx_lens[s] + q_lens[s])
        slots.append(bt[s, t // BS].long() * BS + t % BS)
    T = sum(q_lens)
    dev = torch.device(device)
    query = torch.randn((T, H, D), generator=g, dtype=torch.float32, device=dev).to(dt)
    key = torch.randn((T, KVH, D), generator=g, dtype=torch.float32, device=dev).to(dt)
    value = torch.randn((T, KVH, D), generator=g, dtype=torch.float32, device=dev).to(dt)
    key_cache = torch.randn((pool, KVH, D // x, BS, x), generator=g, dtype=torch.float32, device=dev).to(dt)
    value_cache = torch.randn((pool, KVH, D, BS), generator=g, dtype=torch.float32, device=dev).to(dt)
    slot_mapping = torch.cat(slots) if slots else torch.empty(0, dtype=torch.int64)
    # chunk slots (and unused slots) poisoned: the context is the only valid cache content
    nan = torch.tensor(float("nan"), dtype=dt, device=dev)
    valid = torch.zeros(pool * BS, dtype=torch.bool)
    for s in range(S):
        t = torch.arange(ctx_lens[s])
        valid[(bt[s, t // BS].long() * BS + t % BS)] = True
    inv = (~valid).nonzero().flatten()
    if inv.numel():
        b, o = (inv // BS).to(dev), (inv % BS).to(dev)
        key_cache[b, :, :, o, :] = nan
        value_cache[b, :, :, o] = nan
    qsl = torch.tensor([0] + list(torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).tolist()),
                       dtype=torch.int32)
    return PrefixWorkload(query, key, value, key_cache, value_cache, bt.to(dev), qsl.to(dev),
                          torch.tensor(ctx_lens, dtype=torch.int32).to(dev), slot_mapping.to(dev), KVH, BS,
                          list(ctx_lens), list(q_lens))
