// C ABI of the PagedAttention V2 decode library: argument validation, the
// launch planner, and the two stream-ordered launches.  No host
// synchronisation, no device reads on the host, no allocation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/pav2.h"
#include "pav2_internal.h"
#include "cache.h"
#include "prefix.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int elem_bytes(int dt) {
    switch (dt) {
    case PAV2_F32: return 4;
    case PAV2_F16: return 2;
    case PAV2_BF16: return 2;
    case PAV2_FP8_E4M3: return 1;
    default: return 0;
    }
}

const char *dt_name(int dt) {
    switch (dt) {
    case PAV2_F32: return "f32";
    case PAV2_F16: return "f16";
    case PAV2_BF16: return "bf16";
    case PAV2_FP8_E4M3: return "fp8_e4m3";
    default: return "?";
    }
}

bool supported_head_size(int d) {
    // the head sizes the pages' backend lists as supported
    static const int kSizes[] = {64, 80, 96, 112, 120, 128, 192, 256};
    for (int v : kSizes)
        if (v == d) return true;
    return false;
}

int ilog2_exact(int v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

struct Shape {
    int num_seqs, num_heads, num_kv_heads, head_size, block_size;
    int num_blocks, max_blocks_per_seq, max_num_partitions, max_seq_len;
    int qdt, kvdt;
};

// Shape/dtype checks shared by phase 1 and the full call.
int check_shape(const Shape &s) {
    if (s.num_seqs < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", s.num_seqs);
    if (s.num_heads <= 0 || s.num_kv_heads <= 0)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "num_heads (%d) and num_kv_heads (%d) must be > 0",
                    s.num_heads, s.num_kv_heads);
    if (s.num_heads % s.num_kv_heads)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "num_heads (%d) is not a multiple of num_kv_heads (%d)",
                    s.num_heads, s.num_kv_heads);
    if (elem_bytes(s.qdt) == 0 || s.qdt == PAV2_FP8_E4M3)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "query dtype must be f32, f16 or bf16 (got %d)", s.qdt);
    if (elem_bytes(s.kvdt) == 0)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "unknown kv_cache_dtype %d", s.kvdt);
    if (!supported_head_size(s.head_size))
        return fail(PAV2_ERR_UNSUPPORTED, "head_size %d is not one of 64, 80, 96, 112, 120, 128, 192, 256",
                    s.head_size);
    const int x = 16 / elem_bytes(s.kvdt);
    if (s.head_size % x)
        return fail(PAV2_ERR_UNSUPPORTED, "head_size %d is not a multiple of x = %d for kv dtype %s",
                    s.head_size, x, dt_name(s.kvdt));
    if (s.kvdt != s.qdt && s.kvdt != PAV2_FP8_E4M3)
        return fail(PAV2_ERR_UNSUPPORTED, "query dtype %s with kv dtype %s is not supported",
                    dt_name(s.qdt), dt_name(s.kvdt));
    if (s.block_size < 1 || s.block_size > PAV2_PARTITION_SIZE || PAV2_PARTITION_SIZE % s.block_size)
        return fail(PAV2_ERR_INVALID_ARGUMENT,
                    "block_size %d must divide the 512-token partition (a power of two in [1, 512])",
                    s.block_size);
    if (s.num_blocks <= 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "num_blocks must be > 0");
    if (s.max_seq_len < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0");
    const int need = (s.max_seq_len + PAV2_PARTITION_SIZE - 1) / PAV2_PARTITION_SIZE;
    if (s.max_num_partitions < need || s.max_num_partitions < 1)
        return fail(PAV2_ERR_INVALID_ARGUMENT,
                    "max_num_partitions %d < ceil(max_seq_len / 512) = %d", s.max_num_partitions, need);
    if (s.max_num_partitions > pav2::kMaxPartitions)
        return fail(PAV2_ERR_UNSUPPORTED, "max_num_partitions %d exceeds %d", s.max_num_partitions,
                    pav2::kMaxPartitions);
    const int64_t blocks_need = ((int64_t)s.max_seq_len + s.block_size - 1) / s.block_size;
    if (s.max_blocks_per_seq < blocks_need || s.max_blocks_per_seq < 1)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "max_blocks_per_seq %d < ceil(max_seq_len / block_size) = %lld",
                    s.max_blocks_per_seq, (long long)blocks_need);
    const int64_t work = (int64_t)s.num_seqs * s.num_heads * s.max_num_partitions;
    if (work > (int64_t)1 << 30)
        return fail(PAV2_ERR_UNSUPPORTED, "num_seqs * num_heads * max_num_partitions = %lld is too large",
                    (long long)work);
    return PAV2_OK;
}

void make_plan(const Shape &s, pav2_plan_t *pl) {
    const int gqa = s.num_heads / s.num_kv_heads;
    const int hg = (gqa + pav2::kMaxHeadsPerGroup - 1) / pav2::kMaxHeadsPerGroup;
    const int bs_log2 = ilog2_exact(s.block_size);
    const int64_t work = (int64_t)s.num_seqs * s.num_kv_heads * hg * s.max_num_partitions;
    pl->head_groups = hg;
    pl->waves_per_partition = pav2::kPhase1Waves;
    const bool compact = pav2::phase1_compact(s.num_seqs);
    pl->phase1_workgroups = (int)((work + 7) / 8 * 8);   // dense grid; compact runs min(this, resident)
    pl->phase1_threads = pav2::kPhase1Waves * 64;
    pl->phase1_lds_bytes =
        pav2::phase1_lds_bytes(gqa, s.head_size, pav2::kPhase1Waves, bs_log2, s.num_seqs, compact);
    pl->phase1_compact = compact ? 1 : 0;
    pl->phase1_rounds = compact ? pav2::phase1_compact_rounds(s.num_seqs) : 0;
    pl->phase1_xcd_classes = compact && pav2::phase1_xcd_classes(s.num_seqs, s.num_kv_heads, hg) ? 1 : 0;
    pl->phase2_workgroups =
        pav2::phase2_workgroups((int64_t)s.num_seqs * s.num_heads, s.max_num_partitions, s.head_size, s.qdt);
    {
        const int wpp = pav2::phase2_waves_per_pair(s.max_num_partitions);
        pl->phase2_threads = 64 * (wpp > 4 ? wpp : 4);
    }
    pl->phase2_lds_bytes = pav2::phase2_lds_bytes(s.max_num_partitions, s.head_size, s.qdt);
    pl->use_v1 = pav2::prefer_single_pass((int64_t)s.num_seqs * s.num_kv_heads * hg, s.max_num_partitions) ? 1 : 0;
    pl->v1_workgroups = (int)((int64_t)s.num_seqs * s.num_kv_heads * hg);
    pl->v1_lds_bytes = pav2::phase1_lds_bytes(gqa, s.head_size, pav2::kPhase1Waves, bs_log2, s.num_seqs, false);
}

int launch_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return PAV2_OK;
    if (e == hipErrorInvalidValue)
        return fail(PAV2_ERR_UNSUPPORTED, "%s: no kernel variant for this combination", what);
    return fail(PAV2_ERR_LAUNCH, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// The block-sparse arguments of the V2 op (vert_stride <= 1: dense).
struct Sparse {
    int tp_rank, local_blocks, vert_stride, block_size, sliding_step;
};

int check_sparse(const Sparse &sp, const Shape &sh) {
    if (sp.vert_stride <= 1) return PAV2_OK;
    if (sp.block_size <= 0 || sp.block_size % sh.block_size)
        return fail(PAV2_ERR_INVALID_ARGUMENT,
                    "blocksparse_block_size %d must be a positive multiple of block_size %d", sp.block_size,
                    sh.block_size);
    if (sp.local_blocks < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "blocksparse_local_blocks must be >= 0");
    if (sp.tp_rank < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "tp_rank must be >= 0");
    if (sp.block_size > (1 << 24) || ((int64_t)sp.tp_rank + 1) * sh.num_heads > ((int64_t)1 << 30))
        return fail(PAV2_ERR_UNSUPPORTED, "blocksparse_block_size %d or tp_rank %d too large", sp.block_size,
                    sp.tp_rank);
    return PAV2_OK;
}

int run_phase1(float *exp_sums, float *max_logits, void *tmp_output, const void *query,
               const void *key_cache, const void *value_cache, float scale,
               const int32_t *block_tables, const int32_t *seq_lens, const float *alibi_slopes,
               float k_scale, float v_scale, const Shape &sh, hipStream_t stream,
               const Sparse *sparse = nullptr) {
    pav2_plan_t pl;
    make_plan(sh, &pl);
    pav2::Phase1Params p;
    const bool sp = sparse != nullptr && sparse->vert_stride > 1;
    if (sp) {
        p.tp_rank = sparse->tp_rank;
        p.sp_local_blocks = sparse->local_blocks;
        p.sp_vert_stride = sparse->vert_stride;
        p.sp_block_size = sparse->block_size;
        p.sp_sliding_step = sparse->sliding_step;
        pl.phase1_lds_bytes = pav2::phase1_lds_bytes(sh.num_heads / sh.num_kv_heads, sh.head_size, pav2::kPhase1Waves,
                                                     ilog2_exact(sh.block_size), sh.num_seqs, pl.phase1_compact != 0,
                                                     true);
    }
    p.tmp_out = tmp_output;
    p.exp_sums = exp_sums;
    p.max_logits = max_logits;
    p.query = query;
    p.key_cache = static_cast<const uint8_t *>(key_cache);
    p.value_cache = static_cast<const uint8_t *>(value_cache);
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.alibi = alibi_slopes;
    p.query_start_loc = nullptr;
    p.context_lens = nullptr;
    p.num_seqs = sh.num_seqs;
    p.num_heads = sh.num_heads;
    p.num_kv_heads = sh.num_kv_heads;
    p.gqa = sh.num_heads / sh.num_kv_heads;
    p.head_groups = pl.head_groups;
    p.bs_log2 = ilog2_exact(sh.block_size);
    p.max_blocks_per_seq = sh.max_blocks_per_seq;
    p.max_num_partitions = sh.max_num_partitions;
    p.num_work = sh.num_seqs * sh.num_kv_heads * pl.head_groups * sh.max_num_partitions;
    p.sched = pl.phase1_compact;
    p.compact_rounds = pl.phase1_rounds > 0 ? pl.phase1_rounds : pav2::kPhase1CompactRounds;
    p.xcd_classes = pl.phase1_xcd_classes;
    p.head_stride = (int64_t)sh.head_size * sh.block_size * elem_bytes(sh.kvdt);
    p.blk_stride = p.head_stride * sh.num_kv_heads;
    p.scale_log2 = scale * k_scale * 1.4426950408889634f;
    p.v_scale = v_scale;
    return launch_status(pav2::launch_phase1(p, sh.qdt, sh.kvdt, sh.head_size, pl.waves_per_partition,
                                             pl.phase1_lds_bytes, stream),
                         "phase 1");
}

// Single pass: the phase-1 kernel walks all partitions of each (sequence, kv
// head, head group) and writes the output itself.
int run_v1(void *output, const void *query, const void *key_cache, const void *value_cache, float scale,
           const int32_t *block_tables, const int32_t *seq_lens, const float *alibi_slopes, float k_scale,
           float v_scale, const Shape &sh, hipStream_t stream) {
    pav2_plan_t pl;
    make_plan(sh, &pl);
    pav2::Phase1Params p;
    p.tmp_out = output;
    p.exp_sums = nullptr;
    p.max_logits = nullptr;
    p.query = query;
    p.key_cache = static_cast<const uint8_t *>(key_cache);
    p.value_cache = static_cast<const uint8_t *>(value_cache);
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.alibi = alibi_slopes;
    p.query_start_loc = nullptr;
    p.context_lens = nullptr;
    p.num_seqs = sh.num_seqs;
    p.num_heads = sh.num_heads;
    p.num_kv_heads = sh.num_kv_heads;
    p.gqa = sh.num_heads / sh.num_kv_heads;
    p.head_groups = pl.head_groups;
    p.bs_log2 = ilog2_exact(sh.block_size);
    p.max_blocks_per_seq = sh.max_blocks_per_seq;
    p.max_num_partitions = sh.max_num_partitions;
    p.num_work = pl.v1_workgroups;
    p.sched = 2;
    p.head_stride = (int64_t)sh.head_size * sh.block_size * elem_bytes(sh.kvdt);
    p.blk_stride = p.head_stride * sh.num_kv_heads;
    p.scale_log2 = scale * k_scale * 1.4426950408889634f;
    p.v_scale = v_scale;
    return launch_status(pav2::launch_phase1(p, sh.qdt, sh.kvdt, sh.head_size, pl.waves_per_partition,
                                             pl.v1_lds_bytes, stream),
                         "single pass");
}

int run_phase2(void *output, const float *exp_sums, const float *max_logits, const void *tmp_output,
               const int32_t *seq_lens, int num_seqs, int num_heads, int head_size,
               int max_num_partitions, int odt, hipStream_t stream) {
    pav2::Phase2Params p;
    p.out = output;
    p.exp_sums = exp_sums;
    p.max_logits = max_logits;
    p.tmp_out = tmp_output;
    p.seq_lens = seq_lens;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.max_num_partitions = max_num_partitions;
    const int lds = pav2::phase2_lds_bytes(max_num_partitions, head_size, odt);
    return launch_status(pav2::launch_phase2(p, odt, head_size, pav2::kPhase2Threads, lds, stream),
                         "phase 2");
}

int check_phase1_args(float *exp_sums, float *max_logits, void *tmp_output, const void *query,
                      const void *key_cache, const void *value_cache, const int32_t *block_tables,
                      const int32_t *seq_lens, float scale, float k_scale, float v_scale) {
    if (!exp_sums || !max_logits || !tmp_output || !query || !key_cache || !value_cache ||
        !block_tables || !seq_lens)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!isfinite(scale) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PAV2_ERR_INVALID_ARGUMENT, "scale, k_scale and v_scale must be finite");
    return PAV2_OK;
}

// ---- the allocation-free V2 entry point's workspace -------------------------
//
// pav2_paged_attention_v2_noalloc keeps phase 1's partition workspace
// (tmp_output, exp_sums, max_logits) in this file-scope device array instead
// of caller buffers.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never passes `scratch` itself (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device on that device's first call.
constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Bytes of partition workspace a problem needs in the scratch layout
// [tmp_output | exp_sums | max_logits], each part 256-byte aligned.
size_t noalloc_workspace_bytes(const Shape &sh) {
    const size_t slots = (size_t)sh.num_seqs * sh.num_heads * sh.max_num_partitions;
    return round256(slots * sh.head_size * elem_bytes(sh.qdt)) + 2 * round256(slots * sizeof(float));
}

// The calling thread's current device's copy of `scratch`.
int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PAV2_ERR_LAUNCH, "hipGetDevice: HIP error %d (%s)", (int)e, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PAV2_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(PAV2_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: HIP error %d (%s)", dev, (int)e,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PAV2_OK;
}

}  // namespace

extern "C" {

int pav2_phase1(float *exp_sums, float *max_logits, void *tmp_output, const void *query,
                const void *key_cache, const void *value_cache, int num_kv_heads, float scale,
                const int32_t *block_tables, const int32_t *seq_lens, int block_size,
                int max_seq_len, const float *alibi_slopes, pav2_dtype_t kv_cache_dtype,
                float k_scale, float v_scale, int num_seqs, int num_heads, int head_size,
                int num_blocks, int max_blocks_per_seq, int max_num_partitions,
                pav2_dtype_t query_dtype, pav2_stream_t stream) {
    g_err[0] = 0;
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
             max_blocks_per_seq, max_num_partitions, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    if (num_seqs == 0) return PAV2_OK;
    rc = check_phase1_args(exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                           block_tables, seq_lens, scale, k_scale, v_scale);
    if (rc) return rc;
    return run_phase1(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, scale,
                      block_tables, seq_lens, alibi_slopes, k_scale, v_scale, sh,
                      static_cast<hipStream_t>(stream));
}

int pav2_phase2(void *output, const float *exp_sums, const float *max_logits,
                const void *tmp_output, const int32_t *seq_lens, int num_seqs, int num_heads,
                int head_size, int max_num_partitions, pav2_dtype_t out_dtype,
                pav2_stream_t stream) {
    g_err[0] = 0;
    if (num_seqs < 0 || num_heads <= 0)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 and num_heads > 0");
    if (out_dtype != PAV2_F32 && out_dtype != PAV2_F16 && out_dtype != PAV2_BF16)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "output dtype must be f32, f16 or bf16");
    if (!supported_head_size(head_size))
        return fail(PAV2_ERR_UNSUPPORTED, "head_size %d is not supported", head_size);
    if (max_num_partitions < 1 || max_num_partitions > pav2::kMaxPartitions)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "max_num_partitions %d out of [1, %d]", max_num_partitions,
                    pav2::kMaxPartitions);
    if (num_seqs == 0) return PAV2_OK;
    if (!output || !exp_sums || !max_logits || !tmp_output || !seq_lens)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    return run_phase2(output, exp_sums, max_logits, tmp_output, seq_lens, num_seqs, num_heads, head_size,
                      max_num_partitions, (int)out_dtype, static_cast<hipStream_t>(stream));
}

int pav2_paged_attention_v2(void *output, float *exp_sums, float *max_logits, void *tmp_output,
                            const void *query, const void *key_cache, const void *value_cache,
                            int num_kv_heads, float scale, const int32_t *block_tables,
                            const int32_t *seq_lens, int block_size, int max_seq_len,
                            const float *alibi_slopes, pav2_dtype_t kv_cache_dtype, float k_scale,
                            float v_scale, int num_seqs, int num_heads, int head_size,
                            int num_blocks, int max_blocks_per_seq, int max_num_partitions,
                            pav2_dtype_t query_dtype, pav2_stream_t stream) {
    g_err[0] = 0;
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
             max_blocks_per_seq, max_num_partitions, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    if (num_seqs == 0) return PAV2_OK;
    if (!output) return fail(PAV2_ERR_INVALID_ARGUMENT, "output is NULL");
    rc = check_phase1_args(exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                           block_tables, seq_lens, scale, k_scale, v_scale);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = run_phase1(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, scale,
                    block_tables, seq_lens, alibi_slopes, k_scale, v_scale, sh, st);
    if (rc) return rc;
    return run_phase2(output, exp_sums, max_logits, tmp_output, seq_lens, num_seqs, num_heads,
                      head_size, max_num_partitions, (int)query_dtype, st);
}

int pav2_paged_attention_v2_blocksparse(void *output, float *exp_sums, float *max_logits, void *tmp_output,
                                        const void *query, const void *key_cache, const void *value_cache,
                                        int num_kv_heads, float scale, const int32_t *block_tables,
                                        const int32_t *seq_lens, int block_size, int max_seq_len,
                                        const float *alibi_slopes, pav2_dtype_t kv_cache_dtype, float k_scale,
                                        float v_scale, int tp_rank, int blocksparse_local_blocks,
                                        int blocksparse_vert_stride, int blocksparse_block_size,
                                        int blocksparse_head_sliding_step, int num_seqs, int num_heads,
                                        int head_size, int num_blocks, int max_blocks_per_seq,
                                        int max_num_partitions, pav2_dtype_t query_dtype, pav2_stream_t stream) {
    g_err[0] = 0;
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
             max_blocks_per_seq, max_num_partitions, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    const Sparse sp{tp_rank, blocksparse_local_blocks, blocksparse_vert_stride, blocksparse_block_size,
                    blocksparse_head_sliding_step};
    rc = check_sparse(sp, sh);
    if (rc) return rc;
    if (num_seqs == 0) return PAV2_OK;
    if (!output) return fail(PAV2_ERR_INVALID_ARGUMENT, "output is NULL");
    rc = check_phase1_args(exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                           block_tables, seq_lens, scale, k_scale, v_scale);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = run_phase1(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, scale,
                    block_tables, seq_lens, alibi_slopes, k_scale, v_scale, sh, st, &sp);
    if (rc) return rc;
    return run_phase2(output, exp_sums, max_logits, tmp_output, seq_lens, num_seqs, num_heads,
                      head_size, max_num_partitions, (int)query_dtype, st);
}

int pav2_phase1_blocksparse(float *exp_sums, float *max_logits, void *tmp_output, const void *query,
                            const void *key_cache, const void *value_cache, int num_kv_heads, float scale,
                            const int32_t *block_tables, const int32_t *seq_lens, int block_size, int max_seq_len,
                            const float *alibi_slopes, pav2_dtype_t kv_cache_dtype, float k_scale, float v_scale,
                            int tp_rank, int blocksparse_local_blocks, int blocksparse_vert_stride,
                            int blocksparse_block_size, int blocksparse_head_sliding_step, int num_seqs,
                            int num_heads, int head_size, int num_blocks, int max_blocks_per_seq,
                            int max_num_partitions, pav2_dtype_t query_dtype, pav2_stream_t stream) {
    g_err[0] = 0;
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
             max_blocks_per_seq, max_num_partitions, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    const Sparse sp{tp_rank, blocksparse_local_blocks, blocksparse_vert_stride, blocksparse_block_size,
                    blocksparse_head_sliding_step};
    rc = check_sparse(sp, sh);
    if (rc) return rc;
    if (num_seqs == 0) return PAV2_OK;
    rc = check_phase1_args(exp_sums, max_logits, tmp_output, query, key_cache, value_cache,
                           block_tables, seq_lens, scale, k_scale, v_scale);
    if (rc) return rc;
    return run_phase1(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, scale, block_tables,
                      seq_lens, alibi_slopes, k_scale, v_scale, sh, static_cast<hipStream_t>(stream), &sp);
}

int pav2_paged_attention_v1(void *output, const void *query, const void *key_cache,
                            const void *value_cache, int num_kv_heads, float scale,
                            const int32_t *block_tables, const int32_t *seq_lens, int block_size,
                            int max_seq_len, const float *alibi_slopes, pav2_dtype_t kv_cache_dtype,
                            float k_scale, float v_scale, int num_seqs, int num_heads, int head_size,
                            int num_blocks, int max_blocks_per_seq, pav2_dtype_t query_dtype,
                            pav2_stream_t stream) {
    g_err[0] = 0;
    const int maxp = pav2_max_num_partitions(max_seq_len);
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
             max_blocks_per_seq, maxp > 0 ? maxp : 1, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    if (num_seqs == 0) return PAV2_OK;
    if (!output || !query || !key_cache || !value_cache || !block_tables || !seq_lens)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!isfinite(scale) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PAV2_ERR_INVALID_ARGUMENT, "scale, k_scale and v_scale must be finite");
    return run_v1(output, query, key_cache, value_cache, scale, block_tables, seq_lens, alibi_slopes, k_scale,
                  v_scale, sh, static_cast<hipStream_t>(stream));
}

int pav2_paged_attention_v2_noalloc(void *output, const void *query, const void *key_cache,
                                    const void *value_cache, int num_kv_heads, float scale,
                                    const int32_t *block_tables, const int32_t *seq_lens, int block_size,
                                    int max_seq_len, const float *alibi_slopes, pav2_dtype_t kv_cache_dtype,
                                    float k_scale, float v_scale, int num_seqs, int num_heads, int head_size,
                                    int num_blocks, int max_blocks_per_seq, pav2_dtype_t query_dtype,
                                    pav2_stream_t stream) {
    g_err[0] = 0;
    const int maxp = pav2_max_num_partitions(max_seq_len);
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
             max_blocks_per_seq, maxp > 0 ? maxp : 1, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    if (num_seqs == 0) return PAV2_OK;
    if (!output || !query || !key_cache || !value_cache || !block_tables || !seq_lens)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!isfinite(scale) || !isfinite(k_scale) || !isfinite(v_scale))
        return fail(PAV2_ERR_INVALID_ARGUMENT, "scale, k_scale and v_scale must be finite");
    const size_t need = noalloc_workspace_bytes(sh);
    if (need > kScratchBytes)
        return fail(PAV2_ERR_UNSUPPORTED,
                    "the partition workspace of num_seqs %d x num_heads %d x %d partitions x head_size %d needs "
                    "%zu bytes, beyond the %zu-byte scratch of pav2_paged_attention_v2_noalloc; call "
                    "pav2_paged_attention_v2 with caller-allocated buffers",
                    num_seqs, num_heads, sh.max_num_partitions, head_size, need, kScratchBytes);
    void *base = nullptr;
    rc = scratch_address(&base);
    if (rc) return rc;
    const size_t slots = (size_t)num_seqs * num_heads * sh.max_num_partitions;
    uint8_t *b = static_cast<uint8_t *>(base);
    void *tmp_output = b;
    float *exp_sums = reinterpret_cast<float *>(b + round256(slots * head_size * elem_bytes(query_dtype)));
    float *max_logits = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(exp_sums) + round256(slots * sizeof(float)));
    hipStream_t st = static_cast<hipStream_t>(stream);
    // phase 1 writes every slot's statistics and every used slot's output row;
    // phase 2 reads only those, so nothing left from an earlier call is read
    rc = run_phase1(exp_sums, max_logits, tmp_output, query, key_cache, value_cache, scale, block_tables, seq_lens,
                    alibi_slopes, k_scale, v_scale, sh, st);
    if (rc) return rc;
    return run_phase2(output, exp_sums, max_logits, tmp_output, seq_lens, num_seqs, num_heads, head_size,
                      sh.max_num_partitions, (int)query_dtype, st);
}

size_t pav2_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pav2_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
              int max_num_partitions, pav2_dtype_t query_dtype, pav2_dtype_t kv_cache_dtype,
              pav2_plan_t *plan) {
    g_err[0] = 0;
    if (!plan) return fail(PAV2_ERR_INVALID_ARGUMENT, "plan is NULL");
    const int max_seq_len = max_num_partitions * PAV2_PARTITION_SIZE;
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, 1,
             (max_seq_len + (block_size > 0 ? block_size : 1) - 1) / (block_size > 0 ? block_size : 1),
             max_num_partitions, max_seq_len, (int)query_dtype, (int)kv_cache_dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    make_plan(sh, plan);
    return PAV2_OK;
}

int pav2_decode_kv(const void *src, float *dst, int64_t n, pav2_dtype_t kv_dtype,
                   pav2_dtype_t compute_dtype, pav2_stream_t stream) {
    g_err[0] = 0;
    if (n < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (n == 0) return PAV2_OK;
    if (!src || !dst) return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (elem_bytes(kv_dtype) == 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "unknown kv dtype %d", kv_dtype);
    if (kv_dtype != PAV2_FP8_E4M3) compute_dtype = kv_dtype;
    if (compute_dtype != PAV2_F32 && compute_dtype != PAV2_F16 && compute_dtype != PAV2_BF16)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "compute dtype must be f32, f16 or bf16");
    return launch_status(pav2::launch_decode_kv(src, dst, n, (int)kv_dtype, (int)compute_dtype,
                                                static_cast<hipStream_t>(stream)),
                         "decode_kv");
}

namespace {

// The MFMA prefix kernel's work count and key-range split for a call (the
// same on the workspace query and the call): 0 when the call does not take
// that kernel.
struct PrefixPlan {
    bool mfma = false;
    int64_t row_blocks = 0, work = 0;
    bool offsets32 = false;
    int splits = 1;
};

PrefixPlan plan_prefix(int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size, int num_blocks,
                       int max_query_len, int max_seq_len, float scale, pav2_dtype_t dtype) {
    PrefixPlan pl;
    const int gqa = num_heads / num_kv_heads;
    pl.mfma = pav2::prefix_mfma_supported((int)dtype, head_size, ilog2_exact(block_size), scale);
    const int rows_per_wg = pl.mfma ? pav2::kPrefixMfmaRows : pav2::kPrefixRows;
    pl.row_blocks = ((int64_t)max_query_len * gqa + rows_per_wg - 1) / rows_per_wg;
    pl.work = (int64_t)num_seqs * num_kv_heads * pl.row_blocks;
    if (pl.mfma) {
        const int64_t blk_stride = (int64_t)head_size * block_size * elem_bytes(dtype) * num_kv_heads;
        pl.offsets32 = (int64_t)num_blocks * blk_stride <= ((int64_t)1 << 32);
    }
    return pl;
}

int prefix_impl(void *output, const void *query, const void *key_cache, const void *value_cache,
                const int32_t *block_tables, const int32_t *query_start_loc, const int32_t *context_lens,
                int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size, int num_blocks,
                int max_blocks_per_seq, int max_query_len, int max_seq_len, float scale, pav2_dtype_t dtype,
                void *workspace, size_t workspace_bytes, pav2_stream_t stream) {
    g_err[0] = 0;
    if (dtype == PAV2_FP8_E4M3)
        return fail(PAV2_ERR_UNSUPPORTED, "prefix attention takes f32, f16 or bf16 caches of the query dtype");
    if (max_query_len < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "max_query_len must be >= 0");
    if (max_seq_len < max_query_len)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "max_seq_len %d < max_query_len %d", max_seq_len, max_query_len);
    Shape sh{num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks, max_blocks_per_seq,
             pav2_max_num_partitions(max_seq_len) > 0 ? pav2_max_num_partitions(max_seq_len) : 1, max_seq_len,
             (int)dtype, (int)dtype};
    int rc = check_shape(sh);
    if (rc) return rc;
    const int gqa = num_heads / num_kv_heads;
    const PrefixPlan pl = plan_prefix(num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                      max_query_len, max_seq_len, scale, dtype);
    const bool mfma = pl.mfma;
    const int64_t row_blocks = pl.row_blocks, work = pl.work;
    if (work > ((int64_t)1 << 31) - 1 || row_blocks > ((int64_t)1 << 30))
        return fail(PAV2_ERR_UNSUPPORTED, "num_seqs * num_kv_heads * row blocks = %lld is too large", (long long)work);
    if (work == 0) return PAV2_OK;
    if (!output || !query || !key_cache || !value_cache || !block_tables || !query_start_loc || !context_lens)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (mfma) {
        pav2::PrefixParams q;
        q.out = output;
        q.query = query;
        q.key_cache = static_cast<const uint8_t *>(key_cache);
        q.value_cache = static_cast<const uint8_t *>(value_cache);
        q.block_tables = block_tables;
        q.query_start_loc = query_start_loc;
        q.context_lens = context_lens;
        q.num_seqs = num_seqs;
        q.num_heads = num_heads;
        q.num_kv_heads = num_kv_heads;
        q.gqa = gqa;
        q.row_blocks = (int)row_blocks;
        q.bs_log2 = ilog2_exact(block_size);
        q.max_blocks_per_seq = max_blocks_per_seq;
        q.num_work = (int)work;
        q.head_stride = (int64_t)head_size * block_size * elem_bytes(dtype);
        q.blk_stride = q.head_stride * num_kv_heads;
        q.scale_log2 = scale * 1.4426950408889634f;
        q.offsets32 = pl.offsets32;
        if (workspace) {   // split the key ranges when the workspace holds the partials
            const int sp = work * pav2::kPrefixMaxSplits > ((int64_t)1 << 31) - 1
                               ? 1
                               : pav2::prefix_splits((int)dtype, head_size, q.offsets32, (int)work, max_seq_len);
            if (sp > 1 && workspace_bytes >= pav2::prefix_workspace_bytes(sp, (int)work, head_size)) {
                q.splits = sp;
                q.part = static_cast<float *>(workspace);
            }
        }
        return launch_status(pav2::launch_prefix(q, (int)dtype, head_size, static_cast<hipStream_t>(stream)),
                             "prefix attention");
    }
    pav2::Phase1Params p;
    p.tmp_out = output;
    p.exp_sums = nullptr;
    p.max_logits = nullptr;
    p.query = query;
    p.key_cache = static_cast<const uint8_t *>(key_cache);
    p.value_cache = static_cast<const uint8_t *>(value_cache);
    p.block_tables = block_tables;
    p.seq_lens = nullptr;
    p.alibi = nullptr;
    p.query_start_loc = query_start_loc;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.gqa = gqa;
    p.head_groups = (int)row_blocks;
    p.bs_log2 = ilog2_exact(block_size);
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_num_partitions = sh.max_num_partitions;
    p.num_work = (int)work;
    p.sched = 3;
    p.head_stride = (int64_t)head_size * block_size * elem_bytes(dtype);
    p.blk_stride = p.head_stride * num_kv_heads;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.v_scale = 1.0f;
    // no cross-wavefront partial outputs and no partition-count prefix
    const int lds = pav2::phase1_lds_bytes(0, head_size, pav2::kPhase1Waves, p.bs_log2, num_seqs, false);
    return launch_status(pav2::launch_phase1(p, (int)dtype, (int)dtype, head_size, pav2::kPhase1Waves, lds,
                                             static_cast<hipStream_t>(stream)),
                         "prefix attention");
}

}  // namespace

int pav2_paged_prefix_attention(void *output, const void *query, const void *key_cache,
                                const void *value_cache, const int32_t *block_tables,
                                const int32_t *query_start_loc, const int32_t *context_lens, int num_seqs,
                                int num_heads, int num_kv_heads, int head_size, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_query_len, int max_seq_len, float scale,
                                pav2_dtype_t dtype, pav2_stream_t stream) {
    return prefix_impl(output, query, key_cache, value_cache, block_tables, query_start_loc, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_size, block_size, num_blocks, max_blocks_per_seq, max_query_len,
                       max_seq_len, scale, dtype, nullptr, 0, stream);
}

int pav2_paged_prefix_attention_ws(void *output, const void *query, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *query_start_loc, const int32_t *context_lens, int num_seqs,
                                   int num_heads, int num_kv_heads, int head_size, int block_size, int num_blocks,
                                   int max_blocks_per_seq, int max_query_len, int max_seq_len, float scale,
                                   pav2_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                   pav2_stream_t stream) {
    return prefix_impl(output, query, key_cache, value_cache, block_tables, query_start_loc, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_size, block_size, num_blocks, max_blocks_per_seq, max_query_len,
                       max_seq_len, scale, dtype, workspace, workspace_bytes, stream);
}

size_t pav2_prefix_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                                   int num_blocks, int max_query_len, int max_seq_len, float scale,
                                   pav2_dtype_t dtype) {
    g_err[0] = 0;
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || head_size <= 0 ||
        block_size <= 0 || (block_size & (block_size - 1)) || num_blocks <= 0 || max_query_len <= 0 ||
        max_seq_len < max_query_len || dtype == PAV2_FP8_E4M3)
        return 0;
    const PrefixPlan pl = plan_prefix(num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                      max_query_len, max_seq_len, scale, dtype);
    if (!pl.mfma || pl.work <= 0 || pl.work * pav2::kPrefixMaxSplits > ((int64_t)1 << 31) - 1) return 0;
    const int sp = pav2::prefix_splits((int)dtype, head_size, pl.offsets32, (int)pl.work, max_seq_len);
    return pav2::prefix_workspace_bytes(sp, (int)pl.work, head_size);
}

int pav2_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                           const int64_t *slot_mapping, pav2_dtype_t kv_cache_dtype, float k_scale,
                           float v_scale, int num_tokens, int num_kv_heads, int head_size, int block_size,
                           int num_blocks, pav2_dtype_t input_dtype, pav2_stream_t stream) {
    g_err[0] = 0;
    if (num_tokens < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (num_kv_heads <= 0 || num_blocks <= 0)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "num_kv_heads (%d) and num_blocks (%d) must be > 0", num_kv_heads,
                    num_blocks);
    if (input_dtype != PAV2_F32 && input_dtype != PAV2_F16 && input_dtype != PAV2_BF16)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "input dtype must be f32, f16 or bf16 (got %d)", (int)input_dtype);
    if (kv_cache_dtype != input_dtype && kv_cache_dtype != PAV2_FP8_E4M3)
        return fail(PAV2_ERR_UNSUPPORTED, "kv_cache_dtype %s must be the input dtype %s or fp8_e4m3",
                    dt_name(kv_cache_dtype), dt_name(input_dtype));
    if (!supported_head_size(head_size))
        return fail(PAV2_ERR_UNSUPPORTED, "head_size %d is not one of 64, 80, 96, 112, 120, 128, 192, 256",
                    head_size);
    const int x = 16 / elem_bytes(kv_cache_dtype);
    if (head_size % x != 0)
        return fail(PAV2_ERR_UNSUPPORTED, "head_size %d is not a multiple of x = %d for %s", head_size, x,
                    dt_name(kv_cache_dtype));
    const int bs_log2 = ilog2_exact(block_size);
    if (bs_log2 < 0 || bs_log2 > 9)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "block_size %d must be a power of two in [1, 512]", block_size);
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale))
        return fail(PAV2_ERR_INVALID_ARGUMENT, "k_scale (%g) and v_scale (%g) must be finite and > 0",
                    (double)k_scale, (double)v_scale);
    if (num_tokens == 0) return PAV2_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    pav2::CacheParams p;
    p.key = static_cast<const uint8_t *>(key);
    p.value = static_cast<const uint8_t *>(value);
    p.key_cache = static_cast<uint8_t *>(key_cache);
    p.value_cache = static_cast<uint8_t *>(value_cache);
    p.slot_mapping = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.head_size = head_size;
    p.bs_log2 = bs_log2;
    p.num_slots = (int64_t)num_blocks << bs_log2;
    p.head_stride = (int64_t)head_size * block_size * elem_bytes(kv_cache_dtype);
    p.blk_stride = p.head_stride * num_kv_heads;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.k_rcp = 1.0f / k_scale;
    p.v_rcp = 1.0f / v_scale;
    const auto normal_rcp = [](float sc) { return sc >= 0x1p-100f && sc <= 0x1p100f; };
    p.fast_div = normal_rcp(k_scale) && normal_rcp(v_scale) ? 1 : 0;
    return launch_status(pav2::launch_cache_write(p, (int)input_dtype, (int)kv_cache_dtype,
                                                  static_cast<hipStream_t>(stream)),
                         "reshape_and_cache");
}

int pav2_check_inputs(const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                      int max_blocks_per_seq, int block_size, int num_blocks, int64_t *report,
                      pav2_stream_t stream) {
    g_err[0] = 0;
    if (!report) return fail(PAV2_ERR_INVALID_ARGUMENT, "report is NULL");
    if (num_seqs < 0) return fail(PAV2_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PAV2_ERR_INVALID_ARGUMENT, "max_blocks_per_seq, block_size and num_blocks must be > 0");
    if (num_seqs > 0 && (!block_tables || !seq_lens))
        return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    return launch_status(pav2::launch_check_inputs(block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                                                   block_size, num_blocks, reinterpret_cast<long long *>(report),
                                                   static_cast<hipStream_t>(stream)),
                         "check_inputs");
}

int pav2_read_stream(const void *src, int64_t bytes, int nontemporal, uint32_t *sink, pav2_stream_t stream) {
    g_err[0] = 0;
    if (bytes < 0 || bytes % 16) return fail(PAV2_ERR_INVALID_ARGUMENT, "bytes (%lld) must be a multiple of 16 and >= 0",
                                             (long long)bytes);
    if (bytes == 0) return PAV2_OK;
    if (!src || !sink) return fail(PAV2_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    // four workgroups per compute unit, each sweeping one contiguous slab
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    }
    return launch_status(pav2::launch_read_stream(src, bytes, nontemporal != 0, sink, 4 * cus,
                                                  static_cast<hipStream_t>(stream)),
                         "read_stream");
}

int pav2_max_num_partitions(int max_seq_len) {
    if (max_seq_len <= 0) return 0;
    return (int)(((int64_t)max_seq_len + PAV2_PARTITION_SIZE - 1) / PAV2_PARTITION_SIZE);
}

const char *pav2_last_error(void) { return g_err; }

int pav2_version(void) { return PAV2_VERSION; }

}  // extern "C"
