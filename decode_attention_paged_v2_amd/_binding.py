"""ctypes binding of libpav2.so: argument marshalling only.

Every computation runs in the library's HIP kernels; nothing here computes
attention, and there is no CPU fallback: if the library cannot be loaded the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3
PARTITION_SIZE = 512

_lock = threading.Lock()
_lib = None


class Pav2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pav2 status {status}: {message}")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "phase1_workgroups", "phase1_threads", "phase1_lds_bytes", "head_groups",
        "waves_per_partition", "phase2_workgroups", "phase2_threads", "phase2_lds_bytes",
        "phase1_compact", "use_v1", "v1_workgroups", "v1_lds_bytes", "phase1_rounds",
        "phase1_xcd_classes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


def lib_path() -> str:
    """The library this process loads: $PAV2_LIBRARY if set, else the in-tree build."""
    return os.environ.get("PAV2_LIBRARY") or _build.LIB


def load():
    """Load libpav2.so (building the in-tree one first only if none exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        attn = [P, P, P, P, P, P, P, I, F, P, P, I, I, P, I, F, F, I, I, I, I, I, I, I, P]
        L.pav2_paged_attention_v2.argtypes = attn
        L.pav2_paged_attention_v2.restype = I
        L.pav2_paged_attention_v1.argtypes = [P, P, P, P, I, F, P, P, I, I, P, I, F, F, I, I, I, I, I, I, P]
        L.pav2_paged_attention_v1.restype = I
        L.pav2_paged_attention_v2_blocksparse.argtypes = attn[:17] + [I, I, I, I, I] + attn[17:]
        L.pav2_paged_attention_v2_blocksparse.restype = I
        L.pav2_phase1_blocksparse.argtypes = attn[1:17] + [I, I, I, I, I] + attn[17:]
        L.pav2_phase1_blocksparse.restype = I
        L.pav2_paged_attention_v2_noalloc.argtypes = [P, P, P, P, I, F, P, P, I, I, P, I, F, F, I, I, I, I, I, I, P]
        L.pav2_paged_attention_v2_noalloc.restype = I
        L.pav2_noalloc_scratch_bytes.argtypes = []
        L.pav2_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.pav2_phase1.argtypes = attn[1:]
        L.pav2_phase1.restype = I
        L.pav2_phase2.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
        L.pav2_phase2.restype = I
        L.pav2_plan.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(Plan)]
        L.pav2_plan.restype = I
        L.pav2_decode_kv.argtypes = [P, P, ctypes.c_int64, I, I, P]
        L.pav2_decode_kv.restype = I
        L.pav2_paged_prefix_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P]
        L.pav2_paged_prefix_attention.restype = I
        L.pav2_paged_prefix_attention_ws.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P,
                                                     ctypes.c_size_t, P]
        L.pav2_paged_prefix_attention_ws.restype = I
        L.pav2_prefix_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, F, I]
        L.pav2_prefix_workspace_bytes.restype = ctypes.c_size_t
        L.pav2_reshape_and_cache.argtypes = [P, P, P, P, P, I, F, F, I, I, I, I, I, I, P]
        L.pav2_reshape_and_cache.restype = I
        L.pav2_read_stream.argtypes = [P, ctypes.c_int64, I, P, P]
        L.pav2_read_stream.restype = I
        L.pav2_check_inputs.argtypes = [P, P, I, I, I, I, P, P]
        L.pav2_check_inputs.restype = I
        L.pav2_max_num_partitions.argtypes = [I]
        L.pav2_max_num_partitions.restype = I
        L.pav2_last_error.argtypes = []
        L.pav2_last_error.restype = ctypes.c_char_p
        L.pav2_version.argtypes = []
        L.pav2_version.restype = I
        _lib = L
        return L


def last_error() -> str:
    return load().pav2_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise Pav2Error(rc, last_error())


def version() -> int:
    return load().pav2_version()


def max_num_partitions(max_seq_len: int) -> int:
    return load().pav2_max_num_partitions(int(max_seq_len))


# ---- torch marshalling ------------------------------------------------------

def _dtype_code(t, kv_cache_dtype: str = "auto") -> int:
    import torch
    if kv_cache_dtype not in ("auto", None):
        if kv_cache_dtype in ("fp8", "fp8_e4m3"):
            return FP8_E4M3
        raise ValueError(f"unsupported kv_cache_dtype {kv_cache_dtype!r}")
    table = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
             torch.float8_e4m3fn: FP8_E4M3}
    if t.dtype not in table:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return table[t.dtype]


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (this library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _i32(t, name):
    import torch
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    return _dev(t, name)


def _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens, block_size,
            kv_cache_dtype, alibi_slopes):
    S, H, D = (int(v) for v in query.shape)
    if key_cache.dim() != 5 or value_cache.dim() != 4:
        raise ValueError("key_cache must be 5-D and value_cache 4-D")
    if int(key_cache.shape[1]) != int(num_kv_heads) or int(value_cache.shape[3]) != int(block_size):
        raise ValueError("cache shapes disagree with num_kv_heads / block_size")
    if alibi_slopes is not None:
        import torch
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != H:
            raise ValueError("alibi_slopes must be float32 [num_heads]")
    kvdt = _dtype_code(key_cache, kv_cache_dtype)
    return S, H, D, kvdt


def paged_attention_v2(output, exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                       num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                       alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0,
                       stream=None) -> None:
    """The pages' V2 op: fills output, exp_sums, max_logits, tmp_output in place."""
    L = load()
    S, H, D, kvdt = _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens,
                            block_size, kv_cache_dtype, alibi_slopes)
    rc = L.pav2_paged_attention_v2(
        _dev(output, "output"), _dev(exp_sums, "exp_sums"), _dev(max_logits, "max_logits"),
        _dev(tmp_output, "tmp_output"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), int(num_kv_heads), float(scale),
        _i32(block_tables, "block_tables"), _i32(seq_lens, "seq_lens"), int(block_size),
        int(max_seq_len), _dev(alibi_slopes, "alibi_slopes"), kvdt, float(k_scale), float(v_scale),
        S, H, D, int(key_cache.shape[0]), int(block_tables.shape[1]), int(tmp_output.shape[2]),
        _dtype_code(query), _stream(query, stream))
    _check(rc)


def paged_attention_v2_blocksparse(output, exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                                   num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                                   alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0,
                                   tp_rank=0, blocksparse_local_blocks=0, blocksparse_vert_stride=0,
                                   blocksparse_block_size=64, blocksparse_head_sliding_step=0,
                                   stream=None) -> None:
    """The pages' V2 op with its block-sparse arguments (the pages' defaults;
    blocksparse_vert_stride <= 1 is the dense call)."""
    L = load()
    S, H, D, kvdt = _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens,
                            block_size, kv_cache_dtype, alibi_slopes)
    rc = L.pav2_paged_attention_v2_blocksparse(
        _dev(output, "output"), _dev(exp_sums, "exp_sums"), _dev(max_logits, "max_logits"),
        _dev(tmp_output, "tmp_output"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), int(num_kv_heads), float(scale),
        _i32(block_tables, "block_tables"), _i32(seq_lens, "seq_lens"), int(block_size),
        int(max_seq_len), _dev(alibi_slopes, "alibi_slopes"), kvdt, float(k_scale), float(v_scale),
        int(tp_rank), int(blocksparse_local_blocks), int(blocksparse_vert_stride or 0),
        int(blocksparse_block_size), int(blocksparse_head_sliding_step),
        S, H, D, int(key_cache.shape[0]), int(block_tables.shape[1]), int(tmp_output.shape[2]),
        _dtype_code(query), _stream(query, stream))
    _check(rc)


def paged_attention_v1(output, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                       seq_lens, block_size, max_seq_len, alibi_slopes=None, kv_cache_dtype="auto",
                       k_scale=1.0, v_scale=1.0, stream=None) -> None:
    """The pages' V1 op (single pass): fills output in place."""
    L = load()
    S, H, D, kvdt = _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens,
                            block_size, kv_cache_dtype, alibi_slopes)
    if tuple(output.shape) != (S, H, D) or output.dtype != query.dtype:
        raise ValueError("output must match query in shape and dtype")
    rc = L.pav2_paged_attention_v1(
        _dev(output, "output"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), int(num_kv_heads), float(scale),
        _i32(block_tables, "block_tables"), _i32(seq_lens, "seq_lens"), int(block_size),
        int(max_seq_len), _dev(alibi_slopes, "alibi_slopes"), kvdt, float(k_scale), float(v_scale),
        S, H, D, int(key_cache.shape[0]), int(block_tables.shape[1]), _dtype_code(query),
        _stream(query, stream))
    _check(rc)


def paged_attention_v2_noalloc(output, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                               seq_lens, block_size, max_seq_len, alibi_slopes=None, kv_cache_dtype="auto",
                               k_scale=1.0, v_scale=1.0, stream=None) -> None:
    """V2 with the partition workspace in the library's per-device scratch
    (pav2_paged_attention_v2_noalloc): fills output in place, allocates nothing.
    Calls that overlap on one GPU share that scratch and race."""
    L = load()
    S, H, D, kvdt = _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens,
                            block_size, kv_cache_dtype, alibi_slopes)
    if tuple(output.shape) != (S, H, D) or output.dtype != query.dtype:
        raise ValueError("output must match query in shape and dtype")
    rc = L.pav2_paged_attention_v2_noalloc(
        _dev(output, "output"), _dev(query, "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), int(num_kv_heads), float(scale),
        _i32(block_tables, "block_tables"), _i32(seq_lens, "seq_lens"), int(block_size),
        int(max_seq_len), _dev(alibi_slopes, "alibi_slopes"), kvdt, float(k_scale), float(v_scale),
        S, H, D, int(key_cache.shape[0]), int(block_tables.shape[1]), _dtype_code(query),
        _stream(query, stream))
    _check(rc)


def noalloc_scratch_bytes() -> int:
    return int(load().pav2_noalloc_scratch_bytes())


def phase1(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, num_kv_heads, scale,
           block_tables, seq_lens, block_size, max_seq_len, alibi_slopes=None,
           kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0, stream=None) -> None:
    L = load()
    S, H, D, kvdt = _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens,
                            block_size, kv_cache_dtype, alibi_slopes)
    rc = L.pav2_phase1(
        _dev(exp_sums, "exp_sums"), _dev(max_logits, "max_logits"), _dev(tmp_output, "tmp_output"),
        _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        int(num_kv_heads), float(scale), _i32(block_tables, "block_tables"),
        _i32(seq_lens, "seq_lens"), int(block_size), int(max_seq_len),
        _dev(alibi_slopes, "alibi_slopes"), kvdt, float(k_scale), float(v_scale),
        S, H, D, int(key_cache.shape[0]), int(block_tables.shape[1]), int(tmp_output.shape[2]),
        _dtype_code(query), _stream(query, stream))
    _check(rc)


def phase1_blocksparse(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, num_kv_heads, scale,
                       block_tables, seq_lens, block_size, max_seq_len, alibi_slopes=None,
                       kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0, tp_rank=0, blocksparse_local_blocks=0,
                       blocksparse_vert_stride=0, blocksparse_block_size=64, blocksparse_head_sliding_step=0,
                       stream=None) -> None:
    L = load()
    S, H, D, kvdt = _common(query, key_cache, value_cache, num_kv_heads, block_tables, seq_lens,
                            block_size, kv_cache_dtype, alibi_slopes)
    rc = L.pav2_phase1_blocksparse(
        _dev(exp_sums, "exp_sums"), _dev(max_logits, "max_logits"), _dev(tmp_output, "tmp_output"),
        _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        int(num_kv_heads), float(scale), _i32(block_tables, "block_tables"),
        _i32(seq_lens, "seq_lens"), int(block_size), int(max_seq_len),
        _dev(alibi_slopes, "alibi_slopes"), kvdt, float(k_scale), float(v_scale),
        int(tp_rank), int(blocksparse_local_blocks), int(blocksparse_vert_stride or 0),
        int(blocksparse_block_size), int(blocksparse_head_sliding_step),
        S, H, D, int(key_cache.shape[0]), int(block_tables.shape[1]), int(tmp_output.shape[2]),
        _dtype_code(query), _stream(query, stream))
    _check(rc)


def phase2(output, exp_sums, max_logits, tmp_output, seq_lens, stream=None) -> None:
    L = load()
    S, H, D = (int(v) for v in output.shape)
    rc = L.pav2_phase2(
        _dev(output, "output"), _dev(exp_sums, "exp_sums"), _dev(max_logits, "max_logits"),
        _dev(tmp_output, "tmp_output"), _i32(seq_lens, "seq_lens"), S, H, D,
        int(tmp_output.shape[2]), _dtype_code(output), _stream(output, stream))
    _check(rc)


def plan(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_num_partitions,
         query_dtype: int, kv_cache_dtype: int) -> dict:
    pl = Plan()
    rc = load().pav2_plan(int(num_seqs), int(num_heads), int(num_kv_heads), int(head_size),
                          int(block_size), int(max_num_partitions), int(query_dtype),
                          int(kv_cache_dtype), ctypes.byref(pl))
    _check(rc)
    return pl.as_dict()


def decode_kv(src, compute_dtype=None, stream=None):
    """Widen a device tensor of KV-cache elements to float32 with the kernels' converters."""
    import torch
    kvdt = _dtype_code(src)
    via = kvdt if compute_dtype is None else _dtype_code(torch.empty(0, dtype=compute_dtype))
    dst = torch.empty(src.numel(), dtype=torch.float32, device=src.device)
    rc = load().pav2_decode_kv(_dev(src, "src"), _dev(dst, "dst"), src.numel(), kvdt, via,
                               _stream(src, stream))
    _check(rc)
    return dst.view(src.shape)


def _prefix_args(output, query, key_cache, value_cache, block_tables, query_start_loc, context_lens, scale):
    T, H, D = (int(v) for v in query.shape)
    if tuple(output.shape) != (T, H, D) or output.dtype != query.dtype:
        raise ValueError("output must match query in shape and dtype")
    if key_cache.dim() != 5 or value_cache.dim() != 4:
        raise ValueError("key_cache must be 5-D and value_cache 4-D")
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise ValueError("prefix attention takes caches of the query dtype")
    NB, KVH, bs = int(value_cache.shape[0]), int(value_cache.shape[1]), int(value_cache.shape[3])
    S = int(context_lens.numel())
    if int(query_start_loc.numel()) != S + 1 or int(block_tables.shape[0]) != S:
        raise ValueError("query_start_loc must be [num_seqs + 1] and block_tables [num_seqs, ...]")
    sc = float(D) ** -0.5 if scale is None else float(scale)
    return S, H, KVH, D, bs, NB, sc


def prefix_workspace_bytes(query, key_cache, value_cache, context_lens, max_query_len, max_seq_len,
                           scale=None) -> int:
    """Bytes of workspace paged_prefix_attention splits its key ranges with on
    the current device (pav2_prefix_workspace_bytes); 0 when it would not."""
    T, H, D = (int(v) for v in query.shape)
    NB, KVH, bs = int(value_cache.shape[0]), int(value_cache.shape[1]), int(value_cache.shape[3])
    sc = float(D) ** -0.5 if scale is None else float(scale)
    return int(load().pav2_prefix_workspace_bytes(int(context_lens.numel()), H, KVH, D, bs, NB, int(max_query_len),
                                                   int(max_seq_len), sc, _dtype_code(query)))


def paged_prefix_attention(output, query, key_cache, value_cache, block_tables, query_start_loc,
                           context_lens, max_query_len, max_seq_len, scale=None, stream=None,
                           workspace="auto") -> None:
    """Paged prefix attention (pav2_paged_prefix_attention_ws): the chunks'
    query rows over their context plus the chunk itself (causal), all read
    from the paged cache -- write the chunks' keys / values there first
    (reshape_and_cache).  scale defaults to head_size ** -0.5.  workspace:
    "auto" allocates what prefix_workspace_bytes asks for (torch's caching
    allocator, so it follows the stream), None runs unsplit, or a uint8
    device tensor of at least that size."""
    import torch
    S, H, KVH, D, bs, NB, sc = _prefix_args(output, query, key_cache, value_cache, block_tables, query_start_loc,
                                            context_lens, scale)
    ws, nbytes = None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a tensor')
        nbytes = prefix_workspace_bytes(query, key_cache, value_cache, context_lens, max_query_len, max_seq_len, sc)
        if nbytes:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=query.device)
    elif workspace is not None:
        ws, nbytes = workspace, int(workspace.numel()) * int(workspace.element_size())
    rc = load().pav2_paged_prefix_attention_ws(
        _dev(output, "output"), _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _i32(block_tables, "block_tables"), _i32(query_start_loc, "query_start_loc"),
        _i32(context_lens, "context_lens"), S, H, KVH, D, bs, NB, int(block_tables.shape[1]), int(max_query_len),
        int(max_seq_len), sc, _dtype_code(query), _dev(ws, "workspace") if ws is not None else None, nbytes,
        _stream(query, stream))
    _check(rc)


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, kv_cache_dtype="auto",
                      k_scale=1.0, v_scale=1.0, stream=None) -> None:
    """KV-cache write (pav2_reshape_and_cache): key, value [T, kv_h, d] into the
    paged caches at slot_mapping [T] (int64; negative = no slot)."""
    import torch
    T, KVH, D = (int(v) for v in key.shape)
    if tuple(value.shape) != (T, KVH, D) or value.dtype != key.dtype:
        raise ValueError("value must match key in shape and dtype")
    if key_cache.dim() != 5 or value_cache.dim() != 4:
        raise ValueError("key_cache must be 5-D and value_cache 4-D")
    NB, bs = int(value_cache.shape[0]), int(value_cache.shape[3])
    if int(key_cache.shape[0]) != NB or int(key_cache.shape[1]) != KVH or int(value_cache.shape[1]) != KVH \
            or int(value_cache.shape[2]) != D or int(key_cache.shape[3]) != bs:
        raise ValueError("cache shapes disagree with key [num_tokens, num_kv_heads, head_size]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    kvdt = _dtype_code(key_cache, kv_cache_dtype)
    rc = load().pav2_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(slot_mapping.reshape(-1), "slot_mapping"), kvdt, float(k_scale), float(v_scale), T, KVH, D, bs, NB,
        _dtype_code(key), _stream(key, stream))
    _check(rc)


def read_stream(buf, sink, nontemporal=True, stream=None) -> None:
    """Read every byte of the device tensor `buf` once (pav2_read_stream): a
    measurement aid for achievable read bandwidth (nontemporal) and for
    flushing the caches between timed steps (ordinary loads).  `sink` is a
    device tensor of at least 4 bytes the kernel may write."""
    if buf.numel() * buf.element_size() % 16:
        raise ValueError("buf must hold a multiple of 16 bytes")
    rc = load().pav2_read_stream(_dev(buf, "buf"), buf.numel() * buf.element_size(), 1 if nontemporal else 0,
                                 _dev(sink, "sink"), _stream(buf, stream))
    _check(rc)


def check_inputs(block_tables, seq_lens, block_size, num_blocks, stream=None) -> dict:
    """Run the device-side validator of block tables and sequence lengths and
    return its report (this synchronises with the stream)."""
    import torch
    S, mbps = (int(v) for v in block_tables.shape)
    if tuple(seq_lens.shape) != (S,):
        raise ValueError("seq_lens must have shape [num_seqs]")
    _i32(block_tables, "block_tables")
    _i32(seq_lens, "seq_lens")
    report = torch.empty(4, dtype=torch.int64, device=block_tables.device)
    st = _stream(block_tables, stream)
    rc = load().pav2_check_inputs(_dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, mbps,
                                  int(block_size), int(num_blocks), _dev(report, "report"), st)
    _check(rc)
    if stream is None:
        torch.cuda.current_stream(block_tables.device).synchronize()
    elif hasattr(stream, "synchronize"):
        stream.synchronize()
    else:
        torch.cuda.synchronize(block_tables.device)
    r = [int(v) for v in report.cpu()]
    return {"bad_sequences": r[0], "first_sequence": r[1], "first_column": r[2], "value": r[3]}


def decode(query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, scale,
           block_size, max_seq_len, alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0,
           v_scale=1.0, stream=None):
    """Allocate the outputs and partition buffers (torch) and run both phases.

    Returns (output, exp_sums, max_logits, tmp_output).
    """
    import torch
    S, H, D = (int(v) for v in query.shape)
    P = max(1, max_num_partitions(max_seq_len))
    dev = query.device
    output = torch.empty_like(query)
    exp_sums = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    max_logits = torch.empty_like(exp_sums)
    tmp_output = torch.empty((S, H, P, D), dtype=query.dtype, device=dev)
    paged_attention_v2(output, exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                       num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                       alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream)
    return output, exp_sums, max_logits, tmp_output


def forward_decode(query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, scale,
                   block_size, max_seq_len, alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0,
                   v_scale=1.0, stream=None):
    """Decode attention with the V1 / V2 choice of page "paged_attn.py"
    (forward_decode), taken by the library's planner (``plan()["use_v1"]``).

    Returns the output tensor.
    """
    import torch
    S, H, D = (int(v) for v in query.shape)
    P = max(1, max_num_partitions(max_seq_len))
    kvdt = _dtype_code(key_cache, kv_cache_dtype)
    pl = plan(S, H, num_kv_heads, D, block_size, P, _dtype_code(query), kvdt)
    if pl["use_v1"]:
        output = torch.empty_like(query)
        paged_attention_v1(output, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                           seq_lens, block_size, max_seq_len, alibi_slopes, kv_cache_dtype, k_scale,
                           v_scale, stream)
        return output
    return decode(query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, scale,
                  block_size, max_seq_len, alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream)[0]
