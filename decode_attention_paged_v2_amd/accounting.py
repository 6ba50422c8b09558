"""Algorithmic byte counts of the decode path (measurement bookkeeping).

Phase 1 reads every cached K and V element once per kv head -- 2 * d * b_kv
bytes per (token, kv head), shared by the kv head's query heads -- plus the
query and the block-table entries the sequences use, and writes one
tmp_output row and two float32 statistics per (seq, head, used partition)
plus the statistics of the unused slots.  Phase 2 reads the used partitions'
rows and statistics and writes the output.  The single-pass (V1) kernel reads
what phase 1 reads and writes only the output.
"""
from __future__ import annotations

PARTITION_SIZE = 512


def kv_bytes(lens, num_kv_heads: int, head_size: int, kv_elem_bytes: int) -> int:
    return sum(lens) * num_kv_heads * 2 * head_size * kv_elem_bytes


def phase1_read_bytes(lens, num_heads, num_kv_heads, head_size, block_size, q_elem_bytes,
                      kv_elem_bytes) -> int:
    blocks = sum((L + block_size - 1) // block_size for L in lens)
    return (kv_bytes(lens, num_kv_heads, head_size, kv_elem_bytes)
            + len(lens) * num_heads * head_size * q_elem_bytes + 4 * blocks + 4 * len(lens))


def phase1_write_bytes(lens, num_heads, head_size, q_elem_bytes, max_num_partitions) -> int:
    used_parts = sum((L + PARTITION_SIZE - 1) // PARTITION_SIZE for L in lens)
    return used_parts * num_heads * head_size * q_elem_bytes + 2 * 4 * len(lens) * num_heads * max_num_partitions


def phase1_bytes(lens, num_heads, num_kv_heads, head_size, block_size, q_elem_bytes, kv_elem_bytes,
                 max_num_partitions) -> int:
    return (phase1_read_bytes(lens, num_heads, num_kv_heads, head_size, block_size, q_elem_bytes, kv_elem_bytes)
            + phase1_write_bytes(lens, num_heads, head_size, q_elem_bytes, max_num_partitions))


def phase2_bytes(lens, num_heads, head_size, q_elem_bytes) -> int:
    used_parts = sum((L + PARTITION_SIZE - 1) // PARTITION_SIZE for L in lens)
    S = len(lens)
    return used_parts * num_heads * (head_size * q_elem_bytes + 8) + S * num_heads * head_size * q_elem_bytes + 4 * S


def v1_bytes(lens, num_heads, num_kv_heads, head_size, block_size, q_elem_bytes, kv_elem_bytes) -> int:
    return (phase1_read_bytes(lens, num_heads, num_kv_heads, head_size, block_size, q_elem_bytes, kv_elem_bytes)
            + len(lens) * num_heads * head_size * q_elem_bytes)


def workload_bytes(wl) -> dict:
    """The counts for a generated workload (decode_attention_paged_v2_amd.workloads.Workload)."""
    qb = wl.query.element_size()
    kvb = wl.key_cache.element_size()
    lens = wl.seq_lens_host
    return {
        "kv": kv_bytes(lens, wl.num_kv_heads, wl.head_size, kvb),
        "phase1": phase1_bytes(lens, wl.num_heads, wl.num_kv_heads, wl.head_size, wl.block_size, qb, kvb,
                               wl.max_num_partitions),
        "phase2": phase2_bytes(lens, wl.num_heads, wl.head_size, qb),
        "v1": v1_bytes(lens, wl.num_heads, wl.num_kv_heads, wl.head_size, wl.block_size, qb, kvb),
    }


def spec_bytes(spec) -> dict:
    """The counts for a workload recipe, from its seeded lengths alone (no tensors)."""
    import torch
    from . import workloads as W
    g = torch.Generator()
    g.manual_seed(spec.seed)
    lens = [int(v) for v in spec.lens(g)]
    qb = W.elem_size(W._DT[spec.q_dtype])
    kvb = W.elem_size(W._DT[spec.kv_dtype])
    maxP = max(1, (max(lens) + PARTITION_SIZE - 1) // PARTITION_SIZE)
    used_parts = sum((L + PARTITION_SIZE - 1) // PARTITION_SIZE for L in lens)
    head_groups = -(-(spec.num_heads // spec.num_kv_heads) // 16)
    return {
        # phase-1 work items: (used partition, kv head, group of <= 16 query heads)
        "phase1_items": used_parts * spec.num_kv_heads * head_groups,
        "kv": kv_bytes(lens, spec.num_kv_heads, spec.head_size, kvb),
        "phase1": phase1_bytes(lens, spec.num_heads, spec.num_kv_heads, spec.head_size, spec.block_size,
                               qb, kvb, maxP),
        "phase1_read": phase1_read_bytes(lens, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                         spec.block_size, qb, kvb),
        "phase1_write": phase1_write_bytes(lens, spec.num_heads, spec.head_size, qb, maxP),
        "phase2": phase2_bytes(lens, spec.num_heads, spec.head_size, qb),
        "v1": v1_bytes(lens, spec.num_heads, spec.num_kv_heads, spec.head_size, spec.block_size, qb, kvb),
    }


def blocksparse_attended_tokens(L, heads, num_heads, pattern) -> int:
    """Tokens of a length-L sequence that at least one of `heads` (query-head
    indices within the rank) attends under the block-sparse pattern
    (tp_rank, local_blocks, vert_stride, sparse block size B, sliding step):
    sparse block k of B tokens is attended by head h when it is one of the
    last local_blocks blocks or k = (tp_rank * num_heads + h) * step (mod
    vert_stride).  Counts whole blocks, the last one cut at L."""
    tp, local, vs, B, step = pattern
    if L <= 0:
        return 0
    q = (L - 1) // B
    if vs <= 1:
        return L
    residues = {((tp * num_heads + h) * step) % vs for h in heads}
    blocks = set(range(max(0, q - local + 1), q + 1))
    for r in residues:
        blocks.update(range(r, q + 1, vs))
    return sum(min(B, L - k * B) for k in blocks)


def blocksparse_kv_bytes(lens, num_heads, num_kv_heads, head_size, kv_elem_bytes, pattern) -> int:
    """K/V bytes block-sparse phase 1 must read: per (sequence, kv head, group
    of <= 16 query heads) the tokens some head of the group attends."""
    gqa = num_heads // num_kv_heads
    total = 0
    for L in lens:
        for g in range(num_kv_heads):
            for h0 in range(0, gqa, 16):
                heads = [g * gqa + h0 + r for r in range(min(16, gqa - h0))]
                total += blocksparse_attended_tokens(L, heads, num_heads, pattern)
    return total * 2 * head_size * kv_elem_bytes


def blocksparse_workload_bytes(wl, pattern) -> dict:
    """Algorithmic bytes of block-sparse V2 for a generated workload: the
    attended K/V (per head group), the query and the block-table entries (the
    kernel loads each partition's slice of the table), and phase 1's writes,
    which are those of the dense decode."""
    qb = wl.query.element_size()
    kvb = wl.key_cache.element_size()
    lens = wl.seq_lens_host
    kv = blocksparse_kv_bytes(lens, wl.num_heads, wl.num_kv_heads, wl.head_size, kvb, pattern)
    blocks = sum((L + wl.block_size - 1) // wl.block_size for L in lens)
    reads = kv + len(lens) * wl.num_heads * wl.head_size * qb + 4 * blocks + 4 * len(lens)
    return {"kv": kv, "phase1": reads + phase1_write_bytes(lens, wl.num_heads, wl.head_size, qb,
                                                           wl.max_num_partitions),
            "phase2": phase2_bytes(lens, wl.num_heads, wl.head_size, qb)}


def blocksparse_spec_bytes(spec, pattern) -> dict:
    """spec_bytes with block-sparse phase-1 reads (the attended K/V per kv-head group)."""
    import torch
    from . import workloads as W
    g = torch.Generator()
    g.manual_seed(spec.seed)
    lens = [int(v) for v in spec.lens(g)]
    kvb = W.elem_size(W._DT[spec.kv_dtype])
    out = dict(spec_bytes(spec))
    kv = blocksparse_kv_bytes(lens, spec.num_heads, spec.num_kv_heads, spec.head_size, kvb, pattern)
    out["phase1_read"] = out["phase1_read"] - out["kv"] + kv
    out["phase1"] = out["phase1_read"] + out["phase1_write"]
    out["kv"] = kv
    return out
