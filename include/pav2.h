/*
 * pav2.h -- PagedAttention V2 decode on AMD MI355X (gfx950): C ABI.
 *
 * The operation (page "paged_attention_v2_pytorch.py", function
 * paged_attention_v2_pytorch, and its signature comments): for every sequence
 * s and query head h, single-query attention of query[s, h, :] over the
 * sequence's first seq_lens[s] cached tokens, read through the block table,
 * computed in two phases:
 *
 *   phase 1, per 512-token partition p of the context (partition bounds as in
 *   page "paged_attention_v2_triton.py", part_start / part_end):
 *     z_t        = scale * (q . K_t) + alibi_slopes[h] * t      (t absolute, 0-based)
 *     m_p        = max_t z_t                      -> max_logits[s, h, p]
 *     l_p        = sum_t exp(z_t - m_p)           -> exp_sums[s, h, p]
 *     o_p        = sum_t exp(z_t - m_p) V_t / l_p -> tmp_output[s, h, p, :]
 *   phase 2, the log-sum-exp combine (page 1, "Cross-partition reduction";
 *   page 2, _paged_attn_v2_reduce_kernel):
 *     M = max_p m_p,  w_p = exp(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p.
 *
 * K_t and V_t are the key / value rows of kv head h / (num_heads /
 * num_kv_heads) (grouped-query attention without expanding K/V), gathered from
 * block block_tables[s, t / block_size], slot t % block_size, multiplied by
 * k_scale / v_scale.  tmp_output holds each partition's own normalised output
 * o_p (the reading under which the pages' phase-2 weights give softmax(z) V).
 *
 * Layouts (all row-major, contiguous, device memory owned by the caller):
 *   query        [num_seqs, num_heads, head_size]                  query_dtype
 *   key_cache    [num_blocks, num_kv_heads, head_size/x, block_size, x]
 *                x = 16 / sizeof(kv element): one 16-byte vector holds x
 *                consecutive head-dim elements of one token     kv_cache_dtype
 *   value_cache  [num_blocks, num_kv_heads, head_size, block_size] kv_cache_dtype
 *   block_tables [num_seqs, max_blocks_per_seq] int32 physical block ids;
 *                entries past a sequence's last block are never read
 *   seq_lens     [num_seqs] int32, 0 <= seq_lens[s] <= max_seq_len
 *   alibi_slopes [num_heads] float32, or NULL for no ALiBi
 *   output       [num_seqs, num_heads, head_size]                  query_dtype
 *   exp_sums     [num_seqs, num_heads, max_num_partitions]         float32
 *   max_logits   [num_seqs, num_heads, max_num_partitions]         float32
 *   tmp_output   [num_seqs, num_heads, max_num_partitions, head_size] query_dtype
 *
 * Slots p >= ceil(seq_lens[s] / 512) get max_logits = -inf and exp_sums = 0;
 * their tmp_output rows are left unwritten.  seq_lens[s] == 0 gives a zero
 * output row.
 *
 * Execution: every call is asynchronous on `stream` (a hipStream_t, NULL for
 * the null stream); the library never synchronises the host, never reads
 * device data on the host, and allocates no memory.  Device-side data (block
 * ids < num_blocks, seq_lens <= max_blocks_per_seq * block_size) is not
 * checked.
 *
 * Errors: every entry point returns PAV2_OK (0) or a negative status and
 * launches nothing on failure; pav2_last_error() gives the calling thread's
 * last message.  No C++ exception crosses this interface.
 */
#ifndef PAV2_H
#define PAV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAV2_PARTITION_SIZE 512
#define PAV2_VERSION 10000 /* 1.0.0 */

typedef enum {
    PAV2_F32 = 0,       /* IEEE binary32 */
    PAV2_F16 = 1,       /* IEEE binary16 */
    PAV2_BF16 = 2,      /* bfloat16 */
    PAV2_FP8_E4M3 = 3   /* OCP fp8 E4M3 ("e4m3fn"), KV cache only */
} pav2_dtype_t;

enum {
    PAV2_OK = 0,
    PAV2_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, inconsistent shape */
    PAV2_ERR_UNSUPPORTED = -2,      /* valid but not implemented (dtype pair, head size) */
    PAV2_ERR_LAUNCH = -3            /* the HIP runtime refused a launch */
};

typedef void *pav2_stream_t; /* hipStream_t */

/*
 * Both phases, stream-ordered: phase 1 writes exp_sums, max_logits and
 * tmp_output; phase 2 reads them and writes output.
 *
 * Argument order follows the pages' V2 op (output, exp_sums, max_logits,
 * tmp_output, query, key_cache, value_cache, num_kv_heads, scale,
 * block_tables, seq_lens, block_size, max_seq_len, alibi_slopes,
 * kv_cache_dtype, k_scale, v_scale); the shapes the pages read from tensor
 * metadata follow, then the query dtype and the stream.
 *
 * Supported: head_size in {64, 80, 96, 112, 120, 128, 192, 256} (the pages'
 * supported head sizes) with head_size % x == 0; block_size any divisor of
 * the 512-token partition (1, 2, 4, ..., 512: page "paged_attn.py",
 * forward_decode, asserts 512 % block_size == 0); num_heads % num_kv_heads == 0;
 * (query_dtype, kv_cache_dtype) in {(F32, F32), (F16, F16), (BF16, BF16),
 * (F32, FP8_E4M3), (F16, FP8_E4M3), (BF16, FP8_E4M3)};
 * max_num_partitions >= ceil(max_seq_len / 512) and <= 16384;
 * max_blocks_per_seq >= ceil(max_seq_len / block_size).
 */
int pav2_paged_attention_v2(
    void *output, float *exp_sums, float *max_logits, void *tmp_output,
    const void *query, const void *key_cache, const void *value_cache,
    int num_kv_heads, float scale,
    const int32_t *block_tables, const int32_t *seq_lens,
    int block_size, int max_seq_len,
    const float *alibi_slopes,
    pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int num_seqs, int num_heads, int head_size, int num_blocks,
    int max_blocks_per_seq, int max_num_partitions,
    pav2_dtype_t query_dtype,
    pav2_stream_t stream);

/*
 * Block-sparse PagedAttention V2: pav2_paged_attention_v2 with the V2 op's
 * remaining arguments, tp_rank and the four blocksparse_* ones, in the pages'
 * order (page "paged_attention_v2_pytorch.py", the op's signature; page
 * "paged_attn.py", forward_decode, which takes the block-sparse branch when
 * blocksparse_vert_stride > 1 and asserts that blocksparse_block_size is a
 * multiple of block_size).  The pages give no body; the pattern taken from
 * the names: with B = blocksparse_block_size, key token t lies in sparse
 * block k = t / B and the decode query (position L - 1) in q = (L - 1) / B;
 * query head h, whose index in the whole model is h' = tp_rank * num_heads +
 * h, attends token t < L when
 *     k > q - blocksparse_local_blocks                     (local window), or
 *     (k - h' * blocksparse_head_sliding_step) mod blocksparse_vert_stride == 0
 *                                       (vertical stripes, slid per head).
 * Tokens a head does not attend take no part in its softmax; a partition in
 * which a head attends nothing gets max_logits = -inf, exp_sums = 0 and a
 * zero tmp_output row; a head that attends nothing at all gets a zero output
 * row.  32-token spans that no head of a kv head's group attends are never
 * read.  blocksparse_vert_stride <= 1 is the dense call (the other sparse
 * arguments are then ignored).
 *
 * Errors as pav2_paged_attention_v2, plus PAV2_ERR_INVALID_ARGUMENT for
 * blocksparse_block_size not a positive multiple of block_size, a negative
 * blocksparse_local_blocks or tp_rank (when vert_stride > 1).
 */
int pav2_paged_attention_v2_blocksparse(
    void *output, float *exp_sums, float *max_logits, void *tmp_output,
    const void *query, const void *key_cache, const void *value_cache,
    int num_kv_heads, float scale,
    const int32_t *block_tables, const int32_t *seq_lens,
    int block_size, int max_seq_len,
    const float *alibi_slopes,
    pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int tp_rank, int blocksparse_local_blocks, int blocksparse_vert_stride,
    int blocksparse_block_size, int blocksparse_head_sliding_step,
    int num_seqs, int num_heads, int head_size, int num_blocks,
    int max_blocks_per_seq, int max_num_partitions,
    pav2_dtype_t query_dtype,
    pav2_stream_t stream);

/*
 * PagedAttention V1, the single-pass variant (page "paged_attn.py",
 * forward_decode, which calls it when every sequence fits one partition or
 * when the sequence x head parallelism already fills the device): the same
 * output as pav2_paged_attention_v2, from one launch and with no partition
 * workspace.  One workgroup per (sequence, kv head, group of up to 16 query
 * heads) walks the sequence's 512-token partitions in order, folding each
 * into a running (max, weight sum, weighted output) with the combine of the
 * pages' cross-partition reduction, and writes the normalised output once.
 *
 * Arguments as the pages' V1 op (output, query, key_cache, value_cache,
 * num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
 * alibi_slopes, kv_cache_dtype, k_scale, v_scale), then the shapes, the query
 * dtype and the stream.  Supported combinations as for V2; there is no
 * partition-count limit beyond max_seq_len <= 16384 * 512.
 */
int pav2_paged_attention_v1(
    void *output,
    const void *query, const void *key_cache, const void *value_cache,
    int num_kv_heads, float scale,
    const int32_t *block_tables, const int32_t *seq_lens,
    int block_size, int max_seq_len,
    const float *alibi_slopes,
    pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int num_seqs, int num_heads, int head_size, int num_blocks,
    int max_blocks_per_seq,
    pav2_dtype_t query_dtype,
    pav2_stream_t stream);

/*
 * PagedAttention V2 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same two launches and the same output as
 * pav2_paged_attention_v2, with phase 1's partition workspace (tmp_output,
 * exp_sums, max_logits) held in a library-owned static device array instead
 * of caller buffers.  Arguments as pav2_paged_attention_v1 (the caller passes
 * the inputs and `output` only); max_num_partitions = ceil(max_seq_len / 512).
 *
 * Limit: the workspace, num_seqs * num_heads * max_num_partitions *
 * (head_size * sizeof(query element) + 8) bytes (each of its three parts
 * rounded up to 256 bytes), must fit the scratch of
 * pav2_noalloc_scratch_bytes() = 64 MiB; larger problems return
 * PAV2_ERR_UNSUPPORTED before any HIP call.  Each GPU holds one copy of the
 * scratch from its first call until the process ends (the calling thread's
 * current device, which must be the stream's); this entry point calls no
 * hipMalloc / hipFree.  Every call on one GPU shares that copy: calls that
 * overlap on one GPU (other streams, other threads) race and must be ordered
 * by the caller.  Nothing in it needs clearing between calls (phase 1 writes
 * every slot phase 2 reads).
 */
int pav2_paged_attention_v2_noalloc(
    void *output,
    const void *query, const void *key_cache, const void *value_cache,
    int num_kv_heads, float scale,
    const int32_t *block_tables, const int32_t *seq_lens,
    int block_size, int max_seq_len,
    const float *alibi_slopes,
    pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int num_seqs, int num_heads, int head_size, int num_blocks,
    int max_blocks_per_seq,
    pav2_dtype_t query_dtype,
    pav2_stream_t stream);

/* Size in bytes of pav2_paged_attention_v2_noalloc's per-device scratch. */
size_t pav2_noalloc_scratch_bytes(void);

/*
 * Phase 1 alone (same arguments as pav2_paged_attention_v2 without `output`): writes
 * exp_sums, max_logits and tmp_output.
 */
int pav2_phase1(
    float *exp_sums, float *max_logits, void *tmp_output,
    const void *query, const void *key_cache, const void *value_cache,
    int num_kv_heads, float scale,
    const int32_t *block_tables, const int32_t *seq_lens,
    int block_size, int max_seq_len,
    const float *alibi_slopes,
    pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int num_seqs, int num_heads, int head_size, int num_blocks,
    int max_blocks_per_seq, int max_num_partitions,
    pav2_dtype_t query_dtype,
    pav2_stream_t stream);

/*
 * Block-sparse phase 1 alone (same arguments as
 * pav2_paged_attention_v2_blocksparse without `output`).
 */
int pav2_phase1_blocksparse(
    float *exp_sums, float *max_logits, void *tmp_output,
    const void *query, const void *key_cache, const void *value_cache,
    int num_kv_heads, float scale,
    const int32_t *block_tables, const int32_t *seq_lens,
    int block_size, int max_seq_len,
    const float *alibi_slopes,
    pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int tp_rank, int blocksparse_local_blocks, int blocksparse_vert_stride,
    int blocksparse_block_size, int blocksparse_head_sliding_step,
    int num_seqs, int num_heads, int head_size, int num_blocks,
    int max_blocks_per_seq, int max_num_partitions,
    pav2_dtype_t query_dtype,
    pav2_stream_t stream);

/*
 * Phase 2 alone, the log-sum-exp combine: reads exp_sums, max_logits and
 * tmp_output for partitions p < min(ceil(seq_lens[s]/512), max_num_partitions)
 * and writes output (dtype `out_dtype`, which is also tmp_output's dtype).
 */
int pav2_phase2(
    void *output, const float *exp_sums, const float *max_logits,
    const void *tmp_output, const int32_t *seq_lens,
    int num_seqs, int num_heads, int head_size, int max_num_partitions,
    pav2_dtype_t out_dtype, pav2_stream_t stream);

/* Launch plan the library would use for a problem (host only, no GPU call). */
typedef struct {
    int phase1_workgroups;    /* phase-1 grid size */
    int phase1_threads;       /* threads per phase-1 workgroup */
    int phase1_lds_bytes;     /* dynamic LDS per phase-1 workgroup */
    int head_groups;          /* ceil(gqa / 16): query-head groups per kv head */
    int waves_per_partition;  /* wavefronts sharing one 512-token partition */
    int phase2_workgroups;
    int phase2_threads;
    int phase2_lds_bytes;
    int phase1_compact;       /* 1: phase 1 walks a compact list of used partitions
                                 (grid: min(phase1_workgroups, phase1_rounds
                                 resident rounds)) */
    int use_v1;               /* 1: the single-pass entry point is the faster choice
                                 (every sequence in one partition, or enough
                                 (sequence, kv head) work to fill the chip) */
    int v1_workgroups;        /* single-pass grid: num_seqs * num_kv_heads * head_groups */
    int v1_lds_bytes;         /* dynamic LDS per single-pass workgroup */
    int phase1_rounds;        /* compact schedule: resident rounds of workgroups
                                 (1 from 16 sequences on, else 8; 0 when dense) */
    int phase1_xcd_classes;   /* compact schedule: 1 when each XCD takes whole
                                 (kv head, head group) classes (16 or more
                                 sequences, classes a multiple of 8) */
} pav2_plan_t;

int pav2_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size,
              int block_size, int max_num_partitions,
              pav2_dtype_t query_dtype, pav2_dtype_t kv_cache_dtype,
              pav2_plan_t *plan);

/*
 * Widen n KV-cache elements of `kv_dtype` to float32 on the device with the
 * conversion phase 1 applies when its MFMA operands are `compute_dtype`
 * (the query dtype; only meaningful for FP8_E4M3 caches, which are widened
 * to f32, f16 or bf16 in registers).  src, dst are device pointers.  A test
 * hook for the device-side element decoding.
 */
int pav2_decode_kv(const void *src, float *dst, int64_t n, pav2_dtype_t kv_dtype,
                   pav2_dtype_t compute_dtype, pav2_stream_t stream);

/*
 * Paged prefix attention for chunked prefill (page "paged_attn.py",
 * forward_prefix / _forward_prefix_pytorch): sequence i has context_lens[i]
 * tokens already in the cache and a chunk of new query tokens, rows
 * query_start_loc[i] .. query_start_loc[i+1]-1 of `query`.  Chunk token j
 * (absolute position context_lens[i] + j), head h, attends to the context and
 * to chunk tokens k <= j (causal):
 *
 *   out[q, h] = softmax_t(scale * q . K_t) V_t,  t <= context_lens[i] + j,
 *
 * with K_t, V_t of kv head h / (num_heads / num_kv_heads) read from the paged
 * cache through block_tables[i] (the decode gather).  The chunk's own keys
 * and values must already be in the cache at their positions (written by
 * pav2_reshape_and_cache, as a backend does before attention); for caches of
 * the query dtype with unit scales that is bit for bit the page's reading of
 * them from the key / value tensors.  The page uses scale = head_size^-0.5.
 *
 *   output, query  [total_query_tokens, num_heads, head_size]  dtype
 *   key_cache, value_cache as for decode, dtype (no fp8, no k/v scales)
 *   block_tables [num_seqs, max_blocks_per_seq] int32, covering context + chunk
 *   query_start_loc [num_seqs + 1] int32, context_lens [num_seqs] int32
 *
 * max_query_len >= every chunk's length and max_seq_len >= every context +
 * chunk length (host values sizing the grid and validating the table width).
 * f16 / bf16 with head sizes 64, 96, 128, 192 or 256, blocks of >= 8 tokens
 * and scale > 0 run on MFMA tiles: one workgroup per (sequence, kv head, 128
 * (token, head) rows), the kv head's keys streamed through LDS 64 at a time
 * with a running softmax.  Other cases (f32, other head sizes, blocks of 1,
 * 2 or 4 tokens) run a vector kernel of 64 rows per workgroup.
 * No ALiBi or sliding window (the page's fallback applies neither).
 * Returns 0, or a negative status with pav2_last_error() set.
 */
int pav2_paged_prefix_attention(
    void *output, const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *query_start_loc, const int32_t *context_lens,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    int num_blocks, int max_blocks_per_seq, int max_query_len, int max_seq_len,
    float scale, pav2_dtype_t dtype, pav2_stream_t stream);

/*
 * pav2_paged_prefix_attention with a caller-owned device workspace that lets
 * the MFMA path split each row block's keys into up to 8 contiguous ranges
 * when too few workgroups would fill the device's compute units (each range
 * computes a partial softmax result in float32; a second kernel combines
 * them as the online softmax combines disjoint key sets: the same quantity
 * as the unsplit call, up to float32 rounding).  workspace holds at least
 * pav2_prefix_workspace_bytes(...) bytes for these arguments on the current
 * device, aligned to 16 bytes, and is not read before it is written; a NULL
 * or smaller workspace runs the call unsplit.  It is in use until the call's
 * work on `stream` completes: calls that may overlap need their own.
 */
int pav2_paged_prefix_attention_ws(
    void *output, const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *query_start_loc, const int32_t *context_lens,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    int num_blocks, int max_blocks_per_seq, int max_query_len, int max_seq_len,
    float scale, pav2_dtype_t dtype, void *workspace, size_t workspace_bytes,
    pav2_stream_t stream);

/*
 * Workspace bytes pav2_paged_prefix_attention_ws uses for these arguments on
 * the current device: 0 when the call would not split (or its arguments are
 * invalid; the call itself reports those).  The split count comes from the
 * kernel's occupancy and the device's compute-unit count, so the figure is
 * per device model.
 */
size_t pav2_prefix_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                   int block_size, int num_blocks, int max_query_len, int max_seq_len,
                                   float scale, pav2_dtype_t dtype);

/*
 * KV-cache write (page "paged_attn.py", write_to_paged_cache, which passes
 * key, value, key_cache, value_cache, slot_mapping, kv_cache_dtype, k_scale
 * and v_scale to reshape_and_cache): stores the keys and values of
 * num_tokens new tokens into the paged caches that the decode entry points
 * read.  Token t goes to slot s = slot_mapping[t], i.e. block s / block_size,
 * offset s % block_size:
 *
 *   key_cache  [s / bs, g, i / x, s % bs, i % x] = enc(key  [t, g, i] / k_scale)
 *   value_cache[s / bs, g, i,     s % bs]        = enc(value[t, g, i] / v_scale)
 *
 * The inverse of the decode gather, which multiplies by k_scale / v_scale.
 * The quotient is an IEEE float32 division; enc rounds it to kv_cache_dtype
 * to nearest, ties to even (FP8_E4M3 saturates at +-448 first; NaN stays
 * NaN).  With unit scales and kv_cache_dtype == input_dtype the write copies
 * the input bits.
 *
 *   key, value    [num_tokens, num_kv_heads, head_size] input_dtype (F32, F16, BF16)
 *   key_cache     [num_blocks, num_kv_heads, head_size/x, block_size, x] kv_cache_dtype
 *   value_cache   [num_blocks, num_kv_heads, head_size, block_size]      kv_cache_dtype
 *   slot_mapping  [num_tokens] int64
 *
 * kv_cache_dtype is input_dtype or FP8_E4M3.  A slot < 0 ("no slot", e.g. a
 * padding token) or >= num_blocks * block_size writes nothing.  Two tokens
 * with the same slot leave either one's data there.  head_size and
 * block_size as for the decode entry points; k_scale and v_scale finite and
 * > 0.  num_tokens == 0 launches nothing.  All pointers are device memory
 * owned by the caller; asynchronous on `stream`; allocates nothing.
 */
int pav2_reshape_and_cache(
    const void *key, const void *value, void *key_cache, void *value_cache,
    const int64_t *slot_mapping, pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
    int num_tokens, int num_kv_heads, int head_size, int block_size, int num_blocks,
    pav2_dtype_t input_dtype, pav2_stream_t stream);

/*
 * Debug validator for the device data the decode entry points take on trust:
 * every seq_lens[s] in [0, max_blocks_per_seq * block_size], and every
 * block_tables[s][j] with j < ceil(seq_lens[s] / block_size) in
 * [0, num_blocks).  Writes, asynchronously on `stream`, into `report`
 * (4 int64 in device memory, owned by the caller; read it after the stream
 * has synchronised): report[0] = number of offending sequences,
 * report[1] = the first one (-1 if none), report[2] = its first offending
 * block-table column (-1 when its length is out of range), report[3] = the
 * offending value.  Allocates nothing; returns PAV2_ERR_INVALID_ARGUMENT for
 * null pointers or non-positive sizes, PAV2_ERR_LAUNCH if a launch fails.
 */
int pav2_check_inputs(const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                      int max_blocks_per_seq, int block_size, int num_blocks, int64_t *report,
                      pav2_stream_t stream);

/*
 * Measurement aid, not part of the attention path: read `bytes` (a multiple
 * of 16) of device memory at `src` once with 16-byte vector loads, four
 * workgroups per compute unit each sweeping one contiguous slab.  With
 * nontemporal != 0 the loads carry the streaming hint phase 1 uses for K/V
 * (the chip's achievable read bandwidth for that access); with 0 they are
 * ordinary loads that allocate in L2 and the Infinity Cache, evicting their
 * contents without dirtying them (a cache flush between timed steps).
 * `sink` is one uint32 of caller device memory that the kernel may write.
 * Asynchronous on `stream`; allocates nothing.
 */
int pav2_read_stream(const void *src, int64_t bytes, int nontemporal, uint32_t *sink, pav2_stream_t stream);

/* ceil(max_seq_len / 512): the partition count a sequence of that length needs. */
int pav2_max_num_partitions(int max_seq_len);

/* The calling thread's last error message ("" if none). */
const char *pav2_last_error(void);

int pav2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAV2_H */
