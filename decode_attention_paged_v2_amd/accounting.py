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
