"""Float64 CPU oracle for PagedAttention V2 decode.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product library never does.  It
shares no code with the HIP path.

The arithmetic lives in ``pav2_oracle.c`` (plain C, float64; the KV-cache
write in float32, its working precision), which follows
the page "paged_attention_v2_pytorch.py" (function paged_attention_v2_pytorch)
step by step; see that file's header for the steps and for the one reading
taken (partition outputs are normalised by their own exp-sum).  This module
only marshals arrays into that library and builds it with gcc when the shared
object is missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pav2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# dtype codes understood by the C oracle
F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3
ELEM_SIZE = {F32: 4, F16: 2, BF16: 2, FP8_E4M3: 1}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile pav2_oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-pthread",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int
            F = ctypes.c_float
            lib.oracle_decode.argtypes = [I, P, ctypes.c_int64, P]
            lib.oracle_decode.restype = I
            lib.oracle_paged_attention_v2_blocksparse.argtypes = [
                P, P, P, P,            # out, max_logits, exp_sums, tmp_out
                P, I,                  # query, q_dtype
                P, P, I,               # key_cache, value_cache, kv_dtype
                P, I,                  # block_tables, max_blocks_per_seq
                P, P,                  # seq_lens, alibi_slopes
                I, I, I, I, I,         # num_seqs, num_heads, num_kv_heads, head_size, block_size
                I, F, F, F,            # max_num_partitions, scale, k_scale, v_scale
                I, I, I, I, I,         # tp_rank, local_blocks, vert_stride, sparse block size, sliding step
                P, I]                  # pair_mask, num_threads
            lib.oracle_paged_attention_v2_blocksparse.restype = I
            lib.oracle_dense_attention_blocksparse.argtypes = [
                P,
                P, I,
                P, P, I,
                P, I,
                P, P,
                I, I, I, I, I,
                F, F, F,
                I, I, I, I, I,
                P, I]
            lib.oracle_dense_attention_blocksparse.restype = I
            lib.oracle_encode.argtypes = [I, P, ctypes.c_int64, P]
            lib.oracle_encode.restype = I
            lib.oracle_reshape_and_cache.argtypes = [
                P, P, P, P,            # key, value, key_cache, value_cache
                P, I, F, F,            # slot_mapping, cache_dtype, k_scale, v_scale
                I, I, I, I,            # num_tokens, num_kv_heads, head_size, block_size
                ctypes.c_int64, I]     # num_blocks, input dtype
            lib.oracle_reshape_and_cache.restype = I
            lib.oracle_prefix_attention.argtypes = [
                P, P, I, P, P, P, P, I,   # out, query, q_dtype, key, value, key_cache, value_cache, kv_dtype
                P, I, P, P,               # block_tables, max_blocks_per_seq, query_start_loc, context_lens
                I, I, I, I, I, F]         # num_seqs, num_heads, num_kv_heads, head_size, block_size, scale
            lib.oracle_prefix_attention.restype = I
            _lib = lib
    return _lib


def dtype_code(t) -> int:
    """Map a torch dtype (or a string name) onto the oracle's dtype code."""
    name = str(t).replace("torch.", "")
    table = {"float32": F32, "float16": F16, "bfloat16": BF16,
             "float8_e4m3fn": FP8_E4M3, "f32": F32, "f16": F16, "bf16": BF16,
             "fp8_e4m3": FP8_E4M3}
    if name not in table:
        raise ValueError(f"oracle: unsupported dtype {t}")
    return table[name]


def _raw(t):
    """Contiguous host bytes of a torch tensor or numpy array (kept alive by caller)."""
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t)
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.bfloat16, torch.float8_e4m3fn, torch.float16):
        return t.view(torch.uint8).numpy() if t.dtype == torch.float8_e4m3fn else t.view(torch.int16).numpy()
    return t.numpy()


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def decode(dtype: int, raw: np.ndarray) -> np.ndarray:
    """Widen raw element bytes of the given dtype code to float64, exactly."""
    raw = np.ascontiguousarray(raw)
    n = raw.nbytes // ELEM_SIZE[dtype]
    out = np.empty(n, dtype=np.float64)
    rc = _load().oracle_decode(dtype, _ptr(raw), n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode failed")
    return out


def _threads(n):
    return int(n) if n else (os.cpu_count() or 1)


def _common(query, key_cache, value_cache, block_tables, seq_lens, alibi_slopes):
    q = _raw(query)
    kc = _raw(key_cache)
    vc = _raw(value_cache)
    bt = np.ascontiguousarray(np.asarray(block_tables.cpu() if hasattr(block_tables, "cpu") else block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens, dtype=np.int32))
    al = None
    if alibi_slopes is not None:
        al = np.ascontiguousarray(np.asarray(alibi_slopes.cpu() if hasattr(alibi_slopes, "cpu") else alibi_slopes, dtype=np.float32))
    return q, kc, vc, bt, sl, al


def _sparse_args(tp_rank, local_blocks, vert_stride, bs_block_size, head_sliding_step):
    return (int(tp_rank), int(local_blocks), int(vert_stride or 0), int(bs_block_size), int(head_sliding_step))


def paged_attention_v2(query, key_cache, value_cache, block_tables, seq_lens, *,
                       num_kv_heads, scale, block_size, max_num_partitions,
                       q_dtype, kv_dtype, alibi_slopes=None, k_scale=1.0,
                       v_scale=1.0, pairs=None, threads=None, tp_rank=0,
                       blocksparse_local_blocks=0, blocksparse_vert_stride=0,
                       blocksparse_block_size=64, blocksparse_head_sliding_step=0):
    """Partitioned (V2) decode in float64.

    query [S, H, D]; key_cache [NB, KVH, D/x, BS, x]; value_cache [NB, KVH, D, BS]
    (torch tensors or numpy arrays of raw element bytes); block_tables
    [S, max_blocks_per_seq] int32; seq_lens [S] int32.  ``pairs`` optionally
    lists (s, h) pairs to compute (other rows are returned as NaN).  The
    block-sparse arguments (the V2 op's, with its defaults) select the
    block-sparse pattern when blocksparse_vert_stride > 1 (see
    pav2_oracle.c for the reading taken).

    Returns a dict of float64 arrays: out [S,H,D], max_logits [S,H,P],
    exp_sums [S,H,P], tmp_output [S,H,P,D].
    """
    lib = _load()
    q, kc, vc, bt, sl, al = _common(query, key_cache, value_cache, block_tables, seq_lens, alibi_slopes)
    S, H, D = (int(v) for v in query.shape)
    maxP = int(max_num_partitions)
    out = np.full((S, H, D), np.nan)
    ml = np.full((S, H, maxP), np.nan)
    es = np.full((S, H, maxP), np.nan)
    to = np.full((S, H, maxP, D), np.nan)
    mask = None
    if pairs is not None:
        mask = np.zeros(S * H, dtype=np.uint8)
        for s, h in pairs:
            mask[int(s) * H + int(h)] = 1
    rc = lib.oracle_paged_attention_v2_blocksparse(
        _ptr(out), _ptr(ml), _ptr(es), _ptr(to),
        _ptr(q), q_dtype, _ptr(kc), _ptr(vc), kv_dtype,
        _ptr(bt), bt.shape[1], _ptr(sl), _ptr(al),
        S, H, int(num_kv_heads), D, int(block_size),
        maxP, float(scale), float(k_scale), float(v_scale),
        *_sparse_args(tp_rank, blocksparse_local_blocks, blocksparse_vert_stride, blocksparse_block_size,
                      blocksparse_head_sliding_step),
        _ptr(mask), _threads(threads))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention_v2 rejected its arguments (rc={rc})")
    return {"out": out, "max_logits": ml, "exp_sums": es, "tmp_output": to}


def dense_attention(query, key_cache, value_cache, block_tables, seq_lens, *,
                    num_kv_heads, scale, block_size, q_dtype, kv_dtype,
                    alibi_slopes=None, k_scale=1.0, v_scale=1.0, pairs=None,
                    threads=None, tp_rank=0, blocksparse_local_blocks=0,
                    blocksparse_vert_stride=0, blocksparse_block_size=64,
                    blocksparse_head_sliding_step=0):
    """Unpartitioned decode (one softmax over every attended token) in float64: out [S,H,D]."""
    lib = _load()
    q, kc, vc, bt, sl, al = _common(query, key_cache, value_cache, block_tables, seq_lens, alibi_slopes)
    S, H, D = (int(v) for v in query.shape)
    out = np.full((S, H, D), np.nan)
    mask = None
    if pairs is not None:
        mask = np.zeros(S * H, dtype=np.uint8)
        for s, h in pairs:
            mask[int(s) * H + int(h)] = 1
    rc = lib.oracle_dense_attention_blocksparse(
        _ptr(out), _ptr(q), q_dtype, _ptr(kc), _ptr(vc), kv_dtype,
        _ptr(bt), bt.shape[1], _ptr(sl), _ptr(al),
        S, H, int(num_kv_heads), D, int(block_size),
        float(scale), float(k_scale), float(v_scale),
        *_sparse_args(tp_rank, blocksparse_local_blocks, blocksparse_vert_stride, blocksparse_block_size,
                      blocksparse_head_sliding_step),
        _ptr(mask), _threads(threads))
    if rc != 0:
        raise ValueError(f"oracle_dense_attention rejected its arguments (rc={rc})")
    return out


def encode(dtype: int, values) -> np.ndarray:
    """Round float32 values to elements of the given dtype code (raw element bytes)."""
    src = np.ascontiguousarray(np.asarray(values, dtype=np.float32).ravel())
    out = np.empty(src.size * ELEM_SIZE[dtype], dtype=np.uint8)
    if _load().oracle_encode(dtype, _ptr(src), src.size, _ptr(out)) != 0:
        raise ValueError("oracle_encode failed")
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, block_size,
                      cache_dtype, k_scale=1.0, v_scale=1.0):
    """KV-cache write: key, value [T, kv_h, d] into copies of the paged caches.

    key_cache [NB, kv_h, d/x, block_size, x], value_cache [NB, kv_h, d,
    block_size] are torch tensors or numpy arrays of raw element bytes; the
    caches are not modified.  Returns the written (key_cache, value_cache) as
    numpy arrays of the caches' raw elements (float32; int16 for 16-bit
    formats; uint8 for fp8), in the caches' shapes.
    """
    k = _raw(key)
    v = _raw(value)
    kc = np.array(_raw(key_cache), copy=True)
    vc = np.array(_raw(value_cache), copy=True)
    sm = np.ascontiguousarray(np.asarray(slot_mapping.cpu() if hasattr(slot_mapping, "cpu") else slot_mapping,
                                         dtype=np.int64))
    T, KVH, D = (int(n) for n in key.shape)
    nb = int(key_cache.shape[0])
    in_dtype = dtype_code(key.dtype)
    rc = _load().oracle_reshape_and_cache(
        _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(sm), int(cache_dtype), float(k_scale),
        float(v_scale), T, KVH, D, int(block_size), nb, in_dtype)
    if rc != 0:
        raise ValueError(f"oracle_reshape_and_cache rejected its arguments (rc={rc})")
    return kc, vc


def prefix_attention(query, key, value, key_cache, value_cache, block_tables, query_start_loc,
                     context_lens, *, num_kv_heads, block_size, scale, q_dtype, kv_dtype):
    """Paged prefix attention (chunked prefill) in float64: out [total_q, H, D].

    Context tokens come from the paged caches, the chunk's own keys / values
    from key, value [total_q, kv_h, d] (causal within the chunk)."""
    q = _raw(query)
    k = _raw(key)
    v = _raw(value)
    kc = _raw(key_cache)
    vc = _raw(value_cache)
    i32 = lambda t: np.ascontiguousarray(np.asarray(t.cpu() if hasattr(t, "cpu") else t, dtype=np.int32))
    bt, qsl, cl = i32(block_tables), i32(query_start_loc), i32(context_lens)
    T, H, D = (int(n) for n in query.shape)
    out = np.full((T, H, D), np.nan)
    rc = _load().oracle_prefix_attention(
        _ptr(out), _ptr(q), int(q_dtype), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), int(kv_dtype),
        _ptr(bt), bt.shape[1], _ptr(qsl), _ptr(cl), len(cl), H, int(num_kv_heads), D, int(block_size),
        float(scale))
    if rc != 0:
        raise ValueError(f"oracle_prefix_attention rejected its arguments (rc={rc})")
    return out
