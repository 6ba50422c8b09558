"""C-ABI library checks that need no GPU: it loads, exports every function
include/pav2.h declares, rejects invalid arguments with the documented status
before touching the device, and plans launches on the host."""
import ctypes
import os
import re

import pytest

import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pav2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pav2_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = pav2.load()
    names = declared_functions()
    assert "pav2_paged_attention_v2" in names and len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in pav2.h but not exported"
    assert pav2.version() == 10000


def test_max_num_partitions():
    assert pav2.max_num_partitions(0) == 0
    assert pav2.max_num_partitions(1) == 1
    assert pav2.max_num_partitions(512) == 1
    assert pav2.max_num_partitions(513) == 2
    # 100K context: the page's "195 x bmm" is a floor slip, ceil gives 196
    assert pav2.max_num_partitions(100000) == 196


def _call(**over):
    """pav2_phase1/full call with host-only (null) pointers and overridable sizes."""
    lib = pav2.load()
    a = dict(output=ctypes.c_void_p(16), exp_sums=ctypes.c_void_p(16), max_logits=ctypes.c_void_p(16),
             tmp_output=ctypes.c_void_p(16), query=ctypes.c_void_p(16), key_cache=ctypes.c_void_p(16),
             value_cache=ctypes.c_void_p(16), num_kv_heads=4, scale=0.0625,
             block_tables=ctypes.c_void_p(16), seq_lens=ctypes.c_void_p(16), block_size=16,
             max_seq_len=100000, alibi_slopes=None, kv_cache_dtype=B.BF16, k_scale=1.0, v_scale=1.0,
             num_seqs=4, num_heads=24, head_size=256, num_blocks=25000, max_blocks_per_seq=6250,
             max_num_partitions=196, query_dtype=B.BF16, stream=None)
    a.update(over)
    return lib.pav2_paged_attention_v2(*a.values())


# Each case is invalid, so the call must return before any HIP call.
INVALID = [
    (dict(num_heads=25), -1, "multiple of num_kv_heads"),
    (dict(num_kv_heads=0), -1, "must be > 0"),
    (dict(head_size=100), -2, "head_size 100"),
    (dict(head_size=120, kv_cache_dtype=B.FP8_E4M3), -2, "multiple of x = 16"),
    (dict(block_size=24), -1, "block_size 24"),
    (dict(block_size=1024), -1, "block_size 1024"),
    (dict(block_size=3), -1, "block_size 3"),
    (dict(block_size=0), -1, "block_size 0"),
    (dict(block_size=48), -1, "block_size 48"),
    (dict(max_num_partitions=195), -1, "ceil(max_seq_len / 512) = 196"),
    (dict(max_blocks_per_seq=6249), -1, "max_blocks_per_seq"),
    (dict(query_dtype=B.F16), -2, "query dtype f16 with kv dtype bf16"),
    (dict(query_dtype=B.FP8_E4M3, kv_cache_dtype=B.FP8_E4M3), -1, "query dtype"),
    (dict(kv_cache_dtype=9), -1, "unknown kv_cache_dtype"),
    (dict(output=None), -1, "output is NULL"),
    (dict(query=None), -1, "NULL"),
    (dict(block_tables=None), -1, "NULL"),
    (dict(scale=float("nan")), -1, "finite"),
    (dict(k_scale=float("inf")), -1, "finite"),
    (dict(num_blocks=0), -1, "num_blocks"),
    (dict(max_seq_len=-1), -1, "max_seq_len"),
    (dict(num_seqs=-1), -1, "num_seqs"),
    (dict(max_num_partitions=20000, max_seq_len=20000 * 512, max_blocks_per_seq=640000), -2, "exceeds"),
]


@pytest.mark.parametrize("over,status,msg", INVALID)
def test_invalid_arguments_are_rejected(over, status, msg):
    assert _call(**over) == status
    assert msg in pav2.last_error()


def test_zero_sequences_is_a_no_op():
    assert _call(num_seqs=0, output=None, query=None) == 0
    assert pav2.last_error() == ""


def _call_v1(**over):
    """pav2_paged_attention_v1 with host-only pointers and overridable sizes."""
    lib = pav2.load()
    a = dict(output=ctypes.c_void_p(16), query=ctypes.c_void_p(16), key_cache=ctypes.c_void_p(16),
             value_cache=ctypes.c_void_p(16), num_kv_heads=4, scale=0.0625,
             block_tables=ctypes.c_void_p(16), seq_lens=ctypes.c_void_p(16), block_size=16,
             max_seq_len=100000, alibi_slopes=None, kv_cache_dtype=B.BF16, k_scale=1.0, v_scale=1.0,
             num_seqs=4, num_heads=24, head_size=256, num_blocks=25000, max_blocks_per_seq=6250,
             query_dtype=B.BF16, stream=None)
    a.update(over)
    return lib.pav2_paged_attention_v1(*a.values())


V1_INVALID = [
    (dict(num_heads=25), -1, "multiple of num_kv_heads"),
    (dict(head_size=100), -2, "head_size 100"),
    (dict(block_size=24), -1, "block_size 24"),
    (dict(max_blocks_per_seq=6249), -1, "max_blocks_per_seq"),
    (dict(query_dtype=B.F16), -2, "query dtype f16 with kv dtype bf16"),
    (dict(output=None), -1, "NULL"),
    (dict(seq_lens=None), -1, "NULL"),
    (dict(v_scale=float("nan")), -1, "finite"),
    (dict(max_seq_len=-1), -1, "max_seq_len"),
    (dict(max_seq_len=16385 * 512, max_blocks_per_seq=16385 * 32), -2, "exceeds"),
]


@pytest.mark.parametrize("over,status,msg", V1_INVALID)
def test_v1_invalid_arguments_are_rejected(over, status, msg):
    assert _call_v1(**over) == status
    assert msg in pav2.last_error()


def test_v1_zero_sequences_is_a_no_op():
    assert _call_v1(num_seqs=0, output=None, query=None) == 0
    assert _call_v1(num_seqs=0, max_seq_len=0) == 0
    assert pav2.last_error() == ""


def test_phase2_validation():
    lib = pav2.load()
    v = ctypes.c_void_p(16)
    assert lib.pav2_phase2(v, v, v, v, v, 4, 24, 100, 196, B.BF16, None) == -2
    assert lib.pav2_phase2(v, v, v, v, v, 4, 24, 256, 0, B.BF16, None) == -1
    assert lib.pav2_phase2(v, v, v, v, v, 4, 24, 256, 196, B.FP8_E4M3, None) == -1
    assert lib.pav2_phase2(None, v, v, v, v, 4, 24, 256, 196, B.BF16, None) == -1
    assert lib.pav2_phase2(None, None, None, None, None, 0, 24, 256, 196, B.BF16, None) == 0


def test_check_inputs_validation():
    lib = pav2.load()
    v = ctypes.c_void_p(16)
    assert lib.pav2_check_inputs(v, v, 4, 10, 16, 100, None, None) == -1
    assert "report" in pav2.last_error()
    assert lib.pav2_check_inputs(v, v, -1, 10, 16, 100, v, None) == -1
    assert lib.pav2_check_inputs(v, v, 4, 0, 16, 100, v, None) == -1
    assert lib.pav2_check_inputs(v, v, 4, 10, 16, 0, v, None) == -1
    assert lib.pav2_check_inputs(None, v, 4, 10, 16, 100, v, None) == -1


def test_decode_kv_validation():
    lib = pav2.load()
    v = ctypes.c_void_p(16)
    assert lib.pav2_decode_kv(v, v, -1, B.FP8_E4M3, B.BF16, None) == -1
    assert lib.pav2_decode_kv(None, v, 5, B.FP8_E4M3, B.BF16, None) == -1
    assert lib.pav2_decode_kv(v, v, 5, B.FP8_E4M3, B.FP8_E4M3, None) == -1
    assert lib.pav2_decode_kv(v, v, 0, B.FP8_E4M3, B.BF16, None) == 0


@pytest.mark.parametrize("cfg,expect", [
    # long-context GQA: 4 seqs x 4 kv heads x 196 partitions, 6 query heads per kv head
    (dict(num_seqs=4, num_heads=24, num_kv_heads=4, head_size=256, block_size=16,
          max_num_partitions=196, query_dtype=B.BF16, kv_cache_dtype=B.BF16),
     dict(phase1_workgroups=3136, head_groups=1, phase2_workgroups=96, phase2_threads=1024)),
    # fp8 KV: 64 x 8 x 32
    (dict(num_seqs=64, num_heads=64, num_kv_heads=8, head_size=128, block_size=32,
          max_num_partitions=32, query_dtype=B.BF16, kv_cache_dtype=B.FP8_E4M3),
     dict(phase1_workgroups=16384, head_groups=1, phase2_workgroups=1024)),
    # 32 query heads per kv head need two 16-head groups; grid rounded up to 8
    (dict(num_seqs=3, num_heads=32, num_kv_heads=1, head_size=128, block_size=16,
          max_num_partitions=3, query_dtype=B.F16, kv_cache_dtype=B.F16),
     dict(phase1_workgroups=24, head_groups=2, phase2_workgroups=24)),
])
def test_plan(cfg, expect):
    p = pav2.plan(**cfg)
    for k, v in expect.items():
        assert p[k] == v, (k, p)
    assert p["phase1_threads"] == 256 and p["phase2_threads"] in (256, 1024)
    assert p["phase1_compact"] == (1 if cfg["num_seqs"] > 1 else 0)
    items = cfg["num_seqs"] * cfg["num_kv_heads"] * p["head_groups"]
    assert p["use_v1"] == (1 if items >= 2 * 256 and cfg["max_num_partitions"] <= 32 else 0)
    assert p["v1_workgroups"] == cfg["num_seqs"] * cfg["num_kv_heads"] * p["head_groups"]
    assert p["v1_lds_bytes"] <= p["phase1_lds_bytes"]
    assert 0 < p["phase1_lds_bytes"] <= 160 * 1024
    assert p["phase2_lds_bytes"] == 0
    compact = cfg["num_seqs"] > 1
    assert p["phase1_rounds"] == ((1 if cfg["num_seqs"] >= 16 else 8) if compact else 0)
    assert p["phase1_xcd_classes"] == (1 if compact and cfg["num_seqs"] >= 16 and
                                       (cfg["num_kv_heads"] * p["head_groups"]) % 8 == 0 else 0)


@pytest.mark.parametrize("pairs,maxp,d,odt,expect", [
    (4096, 8, 128, B.F16, 1024),     # one resident round of single-pair wavefronts
    (4097, 8, 128, B.F16, 513),      # two pairs per wavefront: ceil(4097 / 2) waves, 4 per workgroup
    (8192, 64, 80, B.F16, 1024),     # 256 ragged sequences x 32 heads
    (8192, 65, 80, B.F16, 8192),     # 4 wavefronts per pair above 64 partitions: unchanged
    (8192, 8, 256, B.F32, 2048),     # f32 rows of 64 lanes: one pair per wavefront
    (8192, 8, 128, B.F32, 1024),     # f32 rows of 32 lanes fit a half-wavefront
])
def test_plan_phase2_pairs_per_wave(pairs, maxp, d, odt, expect):
    p = pav2.plan(num_seqs=pairs, num_heads=1, num_kv_heads=1, head_size=d, block_size=16,
                  max_num_partitions=maxp, query_dtype=odt, kv_cache_dtype=odt)
    assert p["phase2_workgroups"] == expect


@pytest.mark.parametrize("num_seqs,num_kv_heads,gqa,rounds,classes", [
    (4, 4, 6, 8, 0),      # a few long sequences: 8 resident rounds, items in order
    (15, 8, 4, 8, 0),     # just under the many-sequence bound
    (16, 8, 4, 1, 1),     # many sequences, 8 (kv head, group) classes: one per XCD
    (256, 8, 4, 1, 1),
    (32, 4, 4, 1, 0),     # 4 classes: one round, items in order
    (32, 4, 20, 1, 1),    # 4 kv heads x 2 head groups = 8 classes
    (32, 16, 2, 1, 1),    # 16 classes: two per XCD
    (32, 12, 2, 1, 0),    # 12 classes
])
def test_plan_compact_rounds_and_classes(num_seqs, num_kv_heads, gqa, rounds, classes):
    p = pav2.plan(num_seqs=num_seqs, num_heads=num_kv_heads * gqa, num_kv_heads=num_kv_heads, head_size=128,
                  block_size=16, max_num_partitions=8, query_dtype=B.F16, kv_cache_dtype=B.F16)
    assert (p["phase1_rounds"], p["phase1_xcd_classes"]) == (rounds, classes)


@pytest.mark.parametrize("num_seqs,num_kv_heads,maxp,expect", [
    (1, 4, 1, 1),       # one partition: no combine needed
    (4, 4, 1, 1),
    (256, 8, 4, 1),     # 2048 (seq, kv head) workgroups, 4 partitions each
    (64, 8, 32, 1),     # 512 workgroups = 2 per compute unit, 32 partitions (16K tokens)
    (63, 8, 32, 0),     # just under 2 per compute unit
    (64, 8, 33, 0),     # more than 32 partitions per sequence
    (32, 8, 8, 0),      # 256 workgroups: one per compute unit
    (4, 4, 196, 0),     # long context
])
def test_plan_v1_choice(num_seqs, num_kv_heads, maxp, expect):
    """Single pass when every sequence fits one partition, or when the (seq, kv
    head, head group) workgroups give the 256 compute units two or more each
    and sequences span at most 32 partitions."""
    p = pav2.plan(num_seqs, 8 * num_kv_heads, num_kv_heads, 128, 16, maxp, B.BF16, B.BF16)
    assert p["use_v1"] == expect


def test_python_binding_has_no_cpu_path():
    import torch
    q = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="device tensor"):
        pav2.paged_attention_v2(q, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1), torch.zeros(1, 4, 1, 64),
                                q, torch.zeros(2, 4, 16, 16, 4), torch.zeros(2, 4, 64, 16), 4, 0.125,
                                torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32),
                                16, 1)


def test_reshape_and_cache_validation():
    lib = pav2.load()
    v = ctypes.c_void_p(16)

    def call(**over):
        a = dict(key=v, value=v, key_cache=v, value_cache=v, slot_mapping=v, kv_cache_dtype=B.BF16,
                 k_scale=1.0, v_scale=1.0, num_tokens=4, num_kv_heads=4, head_size=256, block_size=16,
                 num_blocks=100, input_dtype=B.BF16, stream=None)
        a.update(over)
        return lib.pav2_reshape_and_cache(*a.values())
    assert call(num_tokens=-1) == -1
    assert call(num_kv_heads=0) == -1
    assert call(num_blocks=0) == -1
    assert call(input_dtype=B.FP8_E4M3, kv_cache_dtype=B.FP8_E4M3) == -1
    assert call(kv_cache_dtype=B.F16) == -2                       # neither the input dtype nor fp8
    assert call(head_size=100) == -2
    assert call(head_size=120, kv_cache_dtype=B.FP8_E4M3) == -2   # 120 % 16 != 0
    assert call(block_size=24) == -1                              # not a power of two
    assert call(block_size=1024) == -1
    assert call(block_size=0) == -1
    assert call(block_size=4, num_tokens=0) == 0                  # blocks of 1, 2, 4 are accepted
    assert call(k_scale=0.0) == -1
    assert call(v_scale=float("inf")) == -1
    assert call(k_scale=float("nan")) == -1
    assert call(slot_mapping=None) == -1
    assert "NULL" in pav2.last_error()
    # nothing to write: succeeds without a launch, even with null pointers
    assert call(num_tokens=0, key=None, value=None, key_cache=None, value_cache=None, slot_mapping=None) == 0


def test_reshape_and_cache_binding_checks_shapes():
    import torch
    k = torch.zeros(3, 2, 64)
    with pytest.raises(ValueError, match="int64"):
        pav2.reshape_and_cache(k, k, torch.zeros(4, 2, 16, 16, 4), torch.zeros(4, 2, 64, 16),
                               torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="cache shapes"):
        pav2.reshape_and_cache(k, k, torch.zeros(4, 2, 16, 16, 4), torch.zeros(4, 3, 64, 16),
                               torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="device tensor"):
        pav2.reshape_and_cache(k, k, torch.zeros(4, 2, 16, 16, 4), torch.zeros(4, 2, 64, 16),
                               torch.zeros(3, dtype=torch.int64))


def test_prefix_attention_validation():
    lib = pav2.load()
    v = ctypes.c_void_p(16)

    def call(**over):
        a = dict(output=v, query=v, key_cache=v, value_cache=v, block_tables=v, query_start_loc=v,
                 context_lens=v, num_seqs=4, num_heads=24, num_kv_heads=4, head_size=256, block_size=16,
                 num_blocks=1000, max_blocks_per_seq=1100, max_query_len=512, max_seq_len=17000,
                 scale=0.0625, dtype=B.BF16, stream=None)
        a.update(over)
        return lib.pav2_paged_prefix_attention(*a.values())
    assert call(dtype=B.FP8_E4M3) == -2
    assert call(num_heads=25) == -1
    assert call(head_size=100) == -2
    assert call(block_size=24) == -1
    assert call(max_query_len=-1) == -1
    assert call(max_seq_len=100) == -1                 # shorter than the chunk
    assert call(max_blocks_per_seq=10) == -1           # table narrower than ceil(max_seq_len / 16)
    assert call(context_lens=None) == -1
    assert call(num_seqs=0, output=None, query=None) == 0   # nothing to do
    assert call(max_query_len=0, output=None) == 0


def _call_noalloc(**over):
    """pav2_paged_attention_v2_noalloc with host-only pointers and overridable sizes."""
    lib = pav2.load()
    a = dict(output=ctypes.c_void_p(16), query=ctypes.c_void_p(16), key_cache=ctypes.c_void_p(16),
             value_cache=ctypes.c_void_p(16), num_kv_heads=8, scale=0.0625,
             block_tables=ctypes.c_void_p(16), seq_lens=ctypes.c_void_p(16), block_size=16,
             max_seq_len=32768, alibi_slopes=None, kv_cache_dtype=B.F16, k_scale=1.0, v_scale=1.0,
             num_seqs=256, num_heads=32, head_size=80, num_blocks=600000, max_blocks_per_seq=2048,
             query_dtype=B.F16, stream=None)
    a.update(over)
    return lib.pav2_paged_attention_v2_noalloc(*a.values())


def test_noalloc_scratch_limit_is_checked_before_any_hip_call():
    # 256 seqs x 32 heads x 64 partitions x (80 * 2 + 8) bytes = 88 MB of
    # partition workspace does not fit the 64 MiB scratch: rejected up front
    assert pav2.noalloc_scratch_bytes() == 64 << 20
    assert _call_noalloc() == -2
    msg = pav2.last_error()
    assert "scratch" in msg and "pav2_paged_attention_v2 with caller-allocated buffers" in msg
    # the same shape checks as the other entry points
    assert _call_noalloc(num_heads=33) == -1 and "multiple of num_kv_heads" in pav2.last_error()
    assert _call_noalloc(output=None, num_seqs=4) == -1 and "NULL" in pav2.last_error()
    assert _call_noalloc(num_seqs=0, output=None) == 0


def test_noalloc_workspace_bound_is_exact():
    # the largest batch whose workspace fits: tmp rows + two float32 statistics per slot,
    # each part rounded up to 256 bytes
    def need(S, H, P, D, b):
        r = lambda n: (n + 255) // 256 * 256
        return r(S * H * P * D * b) + 2 * r(S * H * P * 4)
    S_fit = max(S for S in range(1, 400) if need(S, 32, 64, 80, 2) <= 64 << 20)
    assert need(S_fit + 1, 32, 64, 80, 2) > 64 << 20
    assert _call_noalloc(num_seqs=S_fit + 1) == -2
