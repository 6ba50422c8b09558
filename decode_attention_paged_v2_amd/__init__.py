"""PagedAttention V2 decode for AMD MI355X (gfx950).

The computation lives in ``libpav2.so`` (hand-written HIP kernels behind the
C ABI declared in ``include/pav2.h``); this package is a thin ctypes binding
whose functions carry the same names as the C entry points.  The library is
loaded on first use; there is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    BF16, F16, F32, FP8_E4M3, PARTITION_SIZE, Pav2Error, check_inputs, decode, decode_kv, forward_decode,
    last_error, lib_path, load, max_num_partitions, noalloc_scratch_bytes, paged_attention_v1, paged_attention_v2,
    paged_attention_v2_blocksparse, paged_attention_v2_noalloc, paged_prefix_attention,
    phase1, phase1_blocksparse, phase2, prefix_workspace_bytes,
    plan, read_stream, reshape_and_cache, version,
)
