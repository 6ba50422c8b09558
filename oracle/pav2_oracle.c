/*
 * pav2_oracle.c -- plain, slow, float64 CPU oracle for PagedAttention V2 decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes, step by step, in the order of the pages (source page
 * "paged_attention_v2_pytorch.py", function paged_attention_v2_pytorch):
 *
 *   0. Unused partition slots: max_logits = -inf, exp_sums = 0, tmp_output = 0
 *      (the "Initialize unused slots" block).
 *   1. seq_len == 0 gives a zero output row (the seq_len == 0 early continue).
 *   2. Paged gather (the "Batched KV gather" block):
 *        block  = block_tables[s, t / block_size]
 *        K[t,i] = key_cache  [block, kv_head, i / x, t % block_size, i % x]
 *        V[t,i] = value_cache[block, kv_head, i,     t % block_size]
 *      then K *= k_scale, V *= v_scale after widening.
 *   3. GQA without expansion: query head h reads kv head h / (H / kv_h)
 *      (the "GQA broadcast" block views q as [kv_h, gqa, 1, d]).
 *   4. Scores z_t = scale * (q . K_t), plus alibi_slopes[h] * t with t the
 *      absolute 0-based position (the "Alibi bias" block).
 *   5. Per 512-token partition p (the padded reshape to [H, P, 512]):
 *        m_p = max z, e_t = exp(z_t - m_p), l_p = sum e_t,
 *        o_p = sum e_t V_t / l_p.
 *      The page stores sum e_t V_t without the division by l_p, but its own
 *      phase-2 combine (and the Triton reduce on page 2) weight the partition
 *      outputs by exp(m_p - M) * l_p / sum, which reproduces softmax(z) V only
 *      for the normalised o_p; the normalised reading is the one taken here.
 *   6. Phase 2 (the "Cross-partition reduction" block):
 *        M = max_p m_p, w_p = exp(m_p - M) * l_p, out = sum_p w_p o_p / sum_p w_p.
 *
 * A second entry point computes the unpartitioned result, one softmax over
 * all tokens (the single-pass online-softmax decode on page 3,
 * "paged_attn.py", _forward_decode_pytorch, reaches the same value), for
 * invariant tests.
 *
 * Block-sparse V2 (the _blocksparse entry points).  The V2 op takes tp_rank
 * and four blocksparse_* arguments (page "paged_attention_v2_pytorch.py",
 * the function's signature; page "paged_attn.py", forward_decode, which takes
 * the block-sparse branch when blocksparse_vert_stride > 1 and requires
 * blocksparse_block_size to be a multiple of the cache block size).  The
 * pages give no body; the reading taken from the names:
 *
 *   B = blocksparse_block_size tokens per sparse block; key token t lies in
 *   sparse block k = t / B, the decode query (position L - 1) in q = (L-1)/B;
 *   h' = tp_rank * num_heads + h is the head's index in the whole model (a
 *   tensor-parallel rank holds num_heads consecutive heads);
 *   query head h attends token t < L iff
 *     k > q - blocksparse_local_blocks                         (local window)
 *     or (k - h' * blocksparse_head_sliding_step) mod vert_stride == 0
 *                                               (vertical stripes, slid per head),
 *   with the modulo taken into [0, vert_stride).  With vert_stride <= 1 the
 *   call is dense.  Scores of tokens a head does not attend are excluded from
 *   its softmax (as the page's -inf padding excludes padded positions);
 *   a partition with no attended token gets max_logits = -inf, exp_sums = 0,
 *   tmp_output = 0 and weight 0 in phase 2; a head with no attended token at
 *   all gets a zero output row, as an empty sequence does.
 *
 * Element decoding is exact widening to double, written from the formats'
 * definitions: IEEE-754 binary32 and binary16, bfloat16 (the upper half of a
 * binary32), and OCP 8-bit E4M3 ("e4m3fn": bias 7, no infinities, S.1111.111
 * is NaN).
 */
#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8_E4M3 = 3 };

#define OR_PARTITION 512

static int elem_size(int dtype) {
    switch (dtype) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    case OR_FP8_E4M3: return 1;
    default: return 0;
    }
}

/* ---- element decoding (exact) ---------------------------------------- */

static double dec_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

static double dec_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static double dec_bf16(uint16_t bits) {
    return dec_f32((uint32_t)bits << 16);
}

static double dec_fp8_e4m3(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xf;
    int m = bits & 0x7;
    double v;
    if (e == 15 && m == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -9);               /* subnormal: (m/8) * 2^-6 */
    } else {
        v = ldexp((double)(8 + m), e - 10);     /* (1 + m/8) * 2^(e-7) */
    }
    return sign ? -v : v;
}

static double dec(int dtype, const void *base, int64_t idx) {
    const uint8_t *p = (const uint8_t *)base;
    switch (dtype) {
    case OR_F32: {
        uint32_t b;
        memcpy(&b, p + 4 * idx, 4);
        return dec_f32(b);
    }
    case OR_F16: {
        uint16_t b;
        memcpy(&b, p + 2 * idx, 2);
        return dec_f16(b);
    }
    case OR_BF16: {
        uint16_t b;
        memcpy(&b, p + 2 * idx, 2);
        return dec_bf16(b);
    }
    case OR_FP8_E4M3:
        return dec_fp8_e4m3(p[idx]);
    default:
        return NAN;
    }
}

/* Decode n elements of one dtype into doubles (exposed so tests can check
 * the decoders against library conversions of every code). */
int oracle_decode(int dtype, const void *src, int64_t n, double *dst) {
    if (elem_size(dtype) == 0) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = dec(dtype, src, i);
    return 0;
}

/* ---- problem description --------------------------------------------- */

typedef struct {
    const void *query;          /* [S, H, D] q_dtype */
    const void *key_cache;      /* [NB, KVH, D/x, BS, x] kv_dtype */
    const void *value_cache;    /* [NB, KVH, D, BS] kv_dtype */
    const int32_t *block_tables;/* [S, MBPS] */
    const int32_t *seq_lens;    /* [S] */
    const float *alibi_slopes;  /* [H] or NULL */
    int q_dtype, kv_dtype;
    int num_seqs, num_heads, num_kv_heads, head_size, block_size;
    int max_blocks_per_seq, max_num_partitions;
    float scale, k_scale, v_scale;
    /* outputs, float64 */
    double *out;                /* [S, H, D] */
    double *max_logits;         /* [S, H, maxP] (partitioned entry only) */
    double *exp_sums;           /* [S, H, maxP] */
    double *tmp_out;            /* [S, H, maxP, D] */
    const uint8_t *pair_mask;   /* [S*H] or NULL: which (s, h) to compute */
    /* block-sparse pattern (vert_stride <= 1: dense) */
    int tp_rank, bs_local_blocks, bs_vert_stride, bs_block_size, bs_head_sliding_step;
    int dense;                  /* 1: unpartitioned softmax, 0: V2 partitioned */
    int next_pair;              /* work counter shared by the threads */
} problem_t;

/* Key element i of logical token t of sequence s, kv head g (step 2). */
static double key_at(const problem_t *P, int s, int g, int t, int i) {
    int x = 16 / elem_size(P->kv_dtype);
    int bs = P->block_size;
    int64_t blk = P->block_tables[(int64_t)s * P->max_blocks_per_seq + t / bs];
    int64_t idx = ((((blk * P->num_kv_heads + g) * (P->head_size / x) + i / x) * bs + t % bs) * x) + i % x;
    return dec(P->kv_dtype, P->key_cache, idx) * (double)P->k_scale;
}

/* Value element i of logical token t of sequence s, kv head g (step 2). */
static double value_at(const problem_t *P, int s, int g, int t, int i) {
    int bs = P->block_size;
    int64_t blk = P->block_tables[(int64_t)s * P->max_blocks_per_seq + t / bs];
    int64_t idx = (((blk * P->num_kv_heads + g) * P->head_size + i) * bs) + t % bs;
    return dec(P->kv_dtype, P->value_cache, idx) * (double)P->v_scale;
}

/* Whether query head h of a sequence of length L attends key token t (the
 * block-sparse reading above; every token when the call is dense). */
static int attended(const problem_t *P, int h, int L, int t) {
    if (P->bs_vert_stride <= 1) return 1;
    int64_t B = P->bs_block_size;
    int64_t k = t / B, q = (L - 1) / B;
    if (k > q - P->bs_local_blocks) return 1;
    int64_t hg = (int64_t)P->tp_rank * P->num_heads + h;
    int64_t r = (k - hg * P->bs_head_sliding_step) % P->bs_vert_stride;
    if (r < 0) r += P->bs_vert_stride;
    return r == 0;
}

/* Scores z_t for t in [0, L) of query head h (steps 3 and 4). */
static void scores(const problem_t *P, int s, int h, int L, double *z) {
    int D = P->head_size;
    int gqa = P->num_heads / P->num_kv_heads;
    int g = h / gqa;
    double slope = P->alibi_slopes ? (double)P->alibi_slopes[h] : 0.0;
    for (int t = 0; t < L; ++t) {
        double dot = 0.0;
        for (int i = 0; i < D; ++i) {
            double q = dec(P->q_dtype, P->query, ((int64_t)s * P->num_heads + h) * D + i);
            dot += q * key_at(P, s, g, t, i);
        }
        z[t] = dot * (double)P->scale;
        if (P->alibi_slopes) z[t] += slope * (double)t;
    }
}

static void solve_pair(const problem_t *P, int s, int h, double *z, double *e) {
    int D = P->head_size;
    int maxP = P->max_num_partitions;
    int gqa = P->num_heads / P->num_kv_heads;
    int g = h / gqa;
    int L = P->seq_lens[s];
    double *out = P->out + ((int64_t)s * P->num_heads + h) * D;

    if (!P->dense) {
        double *ml = P->max_logits + ((int64_t)s * P->num_heads + h) * maxP;
        double *es = P->exp_sums + ((int64_t)s * P->num_heads + h) * maxP;
        double *to = P->tmp_out + ((int64_t)s * P->num_heads + h) * maxP * D;
        /* step 0: every slot starts unused */
        for (int p = 0; p < maxP; ++p) {
            ml[p] = -INFINITY;
            es[p] = 0.0;
            for (int i = 0; i < D; ++i) to[(int64_t)p * D + i] = 0.0;
        }
        if (L == 0) {                                   /* step 1 */
            for (int i = 0; i < D; ++i) out[i] = 0.0;
            return;
        }
        scores(P, s, h, L, z);                          /* steps 2-4 */
        int nparts = (L + OR_PARTITION - 1) / OR_PARTITION;
        for (int p = 0; p < nparts; ++p) {              /* step 5 */
            int t0 = p * OR_PARTITION;
            int t1 = t0 + OR_PARTITION < L ? t0 + OR_PARTITION : L;
            double m = -INFINITY;
            int any = 0;
            for (int t = t0; t < t1; ++t)
                if (attended(P, h, L, t)) {
                    m = z[t] > m ? z[t] : m;
                    any = 1;
                }
            if (!any) continue;                         /* stays -inf / 0 / 0 */
            double l = 0.0;
            for (int t = t0; t < t1; ++t) {
                e[t] = attended(P, h, L, t) ? exp(z[t] - m) : 0.0;
                l += e[t];
            }
            for (int i = 0; i < D; ++i) {
                double acc = 0.0;
                for (int t = t0; t < t1; ++t)
                    if (e[t] != 0.0) acc += e[t] * value_at(P, s, g, t, i);
                to[(int64_t)p * D + i] = acc / l;
            }
            ml[p] = m;
            es[p] = l;
        }
        double M = -INFINITY;                           /* step 6 */
        for (int p = 0; p < nparts; ++p) M = ml[p] > M ? ml[p] : M;
        if (M == -INFINITY) {                           /* no attended token at all */
            for (int i = 0; i < D; ++i) out[i] = 0.0;
            return;
        }
        double W = 0.0;
        for (int p = 0; p < nparts; ++p) W += exp(ml[p] - M) * es[p];
        for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int p = 0; p < nparts; ++p)
                acc += exp(ml[p] - M) * es[p] * to[(int64_t)p * D + i];
            out[i] = acc / W;
        }
    } else {
        if (L == 0) {
            for (int i = 0; i < D; ++i) out[i] = 0.0;
            return;
        }
        scores(P, s, h, L, z);
        double M = -INFINITY;
        for (int t = 0; t < L; ++t)
            if (attended(P, h, L, t)) M = z[t] > M ? z[t] : M;
        if (M == -INFINITY) {
            for (int i = 0; i < D; ++i) out[i] = 0.0;
            return;
        }
        double W = 0.0;
        for (int t = 0; t < L; ++t) {
            e[t] = attended(P, h, L, t) ? exp(z[t] - M) : 0.0;
            W += e[t];
        }
        for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int t = 0; t < L; ++t)
                if (e[t] != 0.0) acc += e[t] * value_at(P, s, g, t, i);
            out[i] = acc / W;
        }
    }
}

static void *worker(void *arg) {
    problem_t *P = (problem_t *)arg;
    int max_len = 0;
    for (int s = 0; s < P->num_seqs; ++s) max_len = P->seq_lens[s] > max_len ? P->seq_lens[s] : max_len;
    double *z = (double *)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double *e = (double *)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    int npairs = P->num_seqs * P->num_heads;
    for (;;) {
        int k = __atomic_fetch_add(&P->next_pair, 1, __ATOMIC_RELAXED);
        if (k >= npairs) break;
        if (P->pair_mask && !P->pair_mask[k]) continue;
        solve_pair(P, k / P->num_heads, k % P->num_heads, z, e);
    }
    free(z);
    free(e);
    return NULL;
}

static int run(problem_t *P, int num_threads) {
    if (elem_size(P->q_dtype) == 0 || elem_size(P->kv_dtype) == 0) return -1;
    if (P->num_kv_heads <= 0 || P->num_heads % P->num_kv_heads != 0) return -1;
    if (P->head_size % (16 / elem_size(P->kv_dtype)) != 0) return -1;
    if (P->block_size <= 0) return -1;
    P->next_pair = 0;
    if (num_threads < 1) num_threads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)num_threads);
    int started = 0;
    for (int k = 1; k < num_threads; ++k)
        if (pthread_create(&th[started], NULL, worker, P) == 0) ++started;
    worker(P);
    for (int k = 0; k < started; ++k) pthread_join(th[k], NULL);
    free(th);
    return 0;
}

static int check_blocksparse(int tp_rank, int local_blocks, int vert_stride, int bs_block_size, int block_size) {
    if (vert_stride <= 1) return 0;
    if (tp_rank < 0 || local_blocks < 0 || bs_block_size <= 0 || bs_block_size % block_size != 0) return -1;
    return 0;
}

/* Partitioned (V2) result: out, max_logits, exp_sums, tmp_out, all float64.
 * pair_mask (optional, [S*H]) restricts the work to selected (s, h) pairs;
 * unselected rows of the outputs are left untouched. */
int oracle_paged_attention_v2_blocksparse(
    double *out, double *max_logits, double *exp_sums, double *tmp_out,
    const void *query, int q_dtype,
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *seq_lens, const float *alibi_slopes,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    int max_num_partitions, float scale, float k_scale, float v_scale,
    int tp_rank, int local_blocks, int vert_stride, int bs_block_size, int head_sliding_step,
    const uint8_t *pair_mask, int num_threads);

int oracle_dense_attention_blocksparse(
    double *out,
    const void *query, int q_dtype,
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *seq_lens, const float *alibi_slopes,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    float scale, float k_scale, float v_scale,
    int tp_rank, int local_blocks, int vert_stride, int bs_block_size, int head_sliding_step,
    const uint8_t *pair_mask, int num_threads);

int oracle_paged_attention_v2_blocksparse(
    double *out, double *max_logits, double *exp_sums, double *tmp_out,
    const void *query, int q_dtype,
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *seq_lens, const float *alibi_slopes,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    int max_num_partitions, float scale, float k_scale, float v_scale,
    int tp_rank, int local_blocks, int vert_stride, int bs_block_size, int head_sliding_step,
    const uint8_t *pair_mask, int num_threads) {
    if (block_size <= 0 || check_blocksparse(tp_rank, local_blocks, vert_stride, bs_block_size, block_size))
        return -1;
    problem_t P;
    memset(&P, 0, sizeof(P));
    P.query = query; P.key_cache = key_cache; P.value_cache = value_cache;
    P.block_tables = block_tables; P.seq_lens = seq_lens; P.alibi_slopes = alibi_slopes;
    P.q_dtype = q_dtype; P.kv_dtype = kv_dtype;
    P.num_seqs = num_seqs; P.num_heads = num_heads; P.num_kv_heads = num_kv_heads;
    P.head_size = head_size; P.block_size = block_size;
    P.max_blocks_per_seq = max_blocks_per_seq; P.max_num_partitions = max_num_partitions;
    P.scale = scale; P.k_scale = k_scale; P.v_scale = v_scale;
    P.out = out; P.max_logits = max_logits; P.exp_sums = exp_sums; P.tmp_out = tmp_out;
    P.pair_mask = pair_mask; P.dense = 0;
    P.tp_rank = tp_rank; P.bs_local_blocks = local_blocks; P.bs_vert_stride = vert_stride;
    P.bs_block_size = bs_block_size; P.bs_head_sliding_step = head_sliding_step;
    for (int s = 0; s < num_seqs; ++s)
        if ((seq_lens[s] + OR_PARTITION - 1) / OR_PARTITION > max_num_partitions) return -2;
    return run(&P, num_threads);
}

int oracle_paged_attention_v2(
    double *out, double *max_logits, double *exp_sums, double *tmp_out,
    const void *query, int q_dtype,
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *seq_lens, const float *alibi_slopes,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    int max_num_partitions, float scale, float k_scale, float v_scale,
    const uint8_t *pair_mask, int num_threads) {
    return oracle_paged_attention_v2_blocksparse(
        out, max_logits, exp_sums, tmp_out, query, q_dtype, key_cache, value_cache, kv_dtype,
        block_tables, max_blocks_per_seq, seq_lens, alibi_slopes, num_seqs, num_heads, num_kv_heads,
        head_size, block_size, max_num_partitions, scale, k_scale, v_scale, 0, 0, 0, 1, 0,
        pair_mask, num_threads);
}

/* Unpartitioned result: one softmax over all (attended) tokens of each (s, h). */
int oracle_dense_attention_blocksparse(
    double *out,
    const void *query, int q_dtype,
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *seq_lens, const float *alibi_slopes,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    float scale, float k_scale, float v_scale,
    int tp_rank, int local_blocks, int vert_stride, int bs_block_size, int head_sliding_step,
    const uint8_t *pair_mask, int num_threads) {
    if (block_size <= 0 || check_blocksparse(tp_rank, local_blocks, vert_stride, bs_block_size, block_size))
        return -1;
    problem_t P;
    memset(&P, 0, sizeof(P));
    P.query = query; P.key_cache = key_cache; P.value_cache = value_cache;
    P.block_tables = block_tables; P.seq_lens = seq_lens; P.alibi_slopes = alibi_slopes;
    P.q_dtype = q_dtype; P.kv_dtype = kv_dtype;
    P.num_seqs = num_seqs; P.num_heads = num_heads; P.num_kv_heads = num_kv_heads;
    P.head_size = head_size; P.block_size = block_size;
    P.max_blocks_per_seq = max_blocks_per_seq;
    P.scale = scale; P.k_scale = k_scale; P.v_scale = v_scale;
    P.out = out; P.pair_mask = pair_mask; P.dense = 1;
    P.tp_rank = tp_rank; P.bs_local_blocks = local_blocks; P.bs_vert_stride = vert_stride;
    P.bs_block_size = bs_block_size; P.bs_head_sliding_step = head_sliding_step;
    return run(&P, num_threads);
}

int oracle_dense_attention(
    double *out,
    const void *query, int q_dtype,
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *seq_lens, const float *alibi_slopes,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    float scale, float k_scale, float v_scale,
    const uint8_t *pair_mask, int num_threads) {
    return oracle_dense_attention_blocksparse(
        out, query, q_dtype, key_cache, value_cache, kv_dtype, block_tables, max_blocks_per_seq,
        seq_lens, alibi_slopes, num_seqs, num_heads, num_kv_heads, head_size, block_size,
        scale, k_scale, v_scale, 0, 0, 0, 1, 0, pair_mask, num_threads);
}

/* ---- KV-cache write ----------------------------------------------------
 *
 * Page "paged_attn.py", write_to_paged_cache: the new tokens' keys and values
 * enter the paged cache through reshape_and_cache(key, value, key_cache,
 * value_cache, slot_mapping, kv_cache_dtype, k_scale, v_scale).  The page
 * shows the call, not its body; the reading taken here is the inverse of the
 * decode gather above (step 2):
 *
 *   slot = slot_mapping[t]; a negative slot means "no slot" and the token is
 *   skipped; block = slot / block_size, offset = slot % block_size;
 *   key_cache  [block, g, i / x, offset, i % x] = enc(key  [t, g, i] / k_scale)
 *   value_cache[block, g, i,     offset]        = enc(value[t, g, i] / v_scale)
 *
 * with x = 16 / element size of the cache dtype (split_kv_cache on the same
 * page).  Decode multiplies by k_scale / v_scale (step 2), so the write
 * divides.  The quotient is taken in float32 (the cache write's working
 * precision, as the scales are float32 arguments), then rounded to the cache
 * dtype to nearest, ties to even.  The cache dtype is the input dtype
 * ("auto") or OCP E4M3; E4M3 saturates at +-448 (it has no infinities), NaN
 * stays NaN.  The encoders below are written from the formats' definitions.
 */

/* Round a > 0 to a binary format with `frac` fraction bits, minimum normal
 * exponent emin, maximum exponent emax and exponent bias `bias` (round to
 * nearest, ties to even: nearbyint in the default rounding mode); returns the
 * code without its sign bit, or -1 when the rounded value overflows. */
static int64_t round_to_format(double a, int frac, int emin, int emax, int bias) {
    if (a == 0.0) return 0;
    int e2;
    frexp(a, &e2);                          /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < emin) {                         /* subnormal grid: multiples of 2^(emin - frac) */
        double m = nearbyint(ldexp(a, frac - emin));
        return (int64_t)m;                  /* m == 2^frac is the smallest normal's code */
    }
    double m = nearbyint(ldexp(a, frac - E));   /* in [2^frac, 2^(frac+1)] */
    if (m == ldexp(1.0, frac + 1)) {
        m = ldexp(1.0, frac);
        E += 1;
    }
    if (E > emax) return -1;
    return ((int64_t)(E + bias) << frac) | ((int64_t)m - ((int64_t)1 << frac));
}

static uint16_t enc_f16(float f) {
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return sign | 0x7e00;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7c00;
    int64_t c = round_to_format(a, 10, -14, 15, 15);
    return c < 0 ? (uint16_t)(sign | 0x7c00) : (uint16_t)(sign | c);
}

static uint16_t enc_bf16(float f) {
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return sign | 0x7fc0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7f80;
    int64_t c = round_to_format(a, 7, -126, 127, 127);
    return c < 0 ? (uint16_t)(sign | 0x7f80) : (uint16_t)(sign | c);
}

static uint8_t enc_fp8_e4m3(float f) {
    double v = (double)f;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v)) return sign | 0x7f;
    double a = fabs(v);
    if (a > 448.0) a = 448.0;               /* saturate (also infinities) */
    int64_t c = round_to_format(a, 3, -6, 8, 7);
    return (uint8_t)(sign | c);             /* c <= 0x7e after saturation */
}

static void store_elem(int dtype, void *base, int64_t idx, float f) {
    uint8_t *p = (uint8_t *)base;
    switch (dtype) {
    case OR_F32: memcpy(p + 4 * idx, &f, 4); break;
    case OR_F16: { uint16_t b = enc_f16(f); memcpy(p + 2 * idx, &b, 2); break; }
    case OR_BF16: { uint16_t b = enc_bf16(f); memcpy(p + 2 * idx, &b, 2); break; }
    case OR_FP8_E4M3: p[idx] = enc_fp8_e4m3(f); break;
    default: break;
    }
}

/* Encode n float32 values into elements of `dtype` (exposed so tests can
 * check the encoders against library conversions). */
int oracle_encode(int dtype, const float *src, int64_t n, void *dst) {
    if (elem_size(dtype) == 0) return -1;
    fesetround(FE_TONEAREST);
    for (int64_t i = 0; i < n; ++i) store_elem(dtype, dst, i, src[i]);
    return 0;
}

int oracle_reshape_and_cache(
    const void *key, const void *value, void *key_cache, void *value_cache,
    const int64_t *slot_mapping, int cache_dtype, float k_scale, float v_scale,
    int num_tokens, int num_kv_heads, int head_size, int block_size,
    int64_t num_blocks, int in_dtype) {
    if (in_dtype == OR_FP8_E4M3 || elem_size(in_dtype) == 0 || elem_size(cache_dtype) == 0) return -1;
    if (cache_dtype != in_dtype && cache_dtype != OR_FP8_E4M3) return -1;
    int x = 16 / elem_size(cache_dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || head_size % x != 0 || block_size <= 0)
        return -1;
    for (int t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= num_blocks * (int64_t)block_size) return -1;
    fesetround(FE_TONEAREST);
    int64_t d = head_size, kvh = num_kv_heads, bs = block_size;
    for (int t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t blk = slot / bs, off = slot % bs;
        for (int64_t g = 0; g < kvh; ++g) {
            for (int64_t i = 0; i < d; ++i) {
                int64_t src = ((int64_t)t * kvh + g) * d + i;
                float kq = (float)dec(in_dtype, key, src) / k_scale;
                float vq = (float)dec(in_dtype, value, src) / v_scale;
                int64_t kidx = (((blk * kvh + g) * (d / x) + i / x) * bs + off) * x + i % x;
                int64_t vidx = ((blk * kvh + g) * d + i) * bs + off;
                store_elem(cache_dtype, key_cache, kidx, kq);
                store_elem(cache_dtype, value_cache, vidx, vq);
            }
        }
    }
    return 0;
}

/* ---- Paged prefix attention (chunked prefill) ----------------------------
 *
 * Page "paged_attn.py", _forward_prefix_pytorch: sequence i has context_lens[i]
 * tokens already in the paged cache and a chunk of q_len_i new tokens
 * (query rows query_start_loc[i] .. query_start_loc[i+1]-1).  Query token j
 * of the chunk (absolute position ctx + j), head h, attends to every context
 * token (all precede it) and to chunk tokens k <= j (the causal mask), with
 * scores q . K * scale, softmax over all of them, times V.  The page streams
 * the keys in tiles with an online softmax; that reaches exactly one softmax
 * over all keys, which is what is computed here.  Context keys come from the
 * cache (block_tables[i][t / bs], slot t % bs, the decode gather), chunk keys
 * from key / value [total_q, kv_h, d]; kv head h / (H / kv_h).  The page uses
 * scale = head_size^-0.5, no scales for the cache and no ALiBi.
 */
int oracle_prefix_attention(
    double *out,                                   /* [total_q, H, D] */
    const void *query, int q_dtype,                /* [total_q, H, D] */
    const void *key, const void *value,            /* [total_q, KVH, D], q_dtype */
    const void *key_cache, const void *value_cache, int kv_dtype,
    const int32_t *block_tables, int max_blocks_per_seq,
    const int32_t *query_start_loc, const int32_t *context_lens,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
    float scale) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return -1;
    if (elem_size(kv_dtype) == 0 || elem_size(q_dtype) == 0 || block_size <= 0) return -1;
    const int D = head_size, H = num_heads, KVH = num_kv_heads, gqa = H / KVH;
    const int x = 16 / elem_size(kv_dtype);
    if (D % x) return -1;
    for (int i = 0; i < num_seqs; ++i) {
        const int q0 = query_start_loc[i], ql = query_start_loc[i + 1] - q0, ctx = context_lens[i];
        if (ql < 0 || ctx < 0) return -1;
        const int nk = ctx + ql;
        double *z = (double *)malloc(sizeof(double) * (nk > 0 ? nk : 1));
        if (!z) return -2;
        for (int j = 0; j < ql; ++j) {
            for (int h = 0; h < H; ++h) {
                const int g = h / gqa, L = ctx + j + 1;
                double m = -INFINITY;
                for (int t = 0; t < L; ++t) {
                    double dot = 0.0;
                    for (int i2 = 0; i2 < D; ++i2) {
                        double q = dec(q_dtype, query, ((int64_t)(q0 + j) * H + h) * D + i2);
                        double k;
                        if (t < ctx) {
                            int64_t blk = block_tables[(int64_t)i * max_blocks_per_seq + t / block_size];
                            k = dec(kv_dtype, key_cache,
                                    (((blk * KVH + g) * (D / x) + i2 / x) * block_size + t % block_size) * x + i2 % x);
                        } else {
                            k = dec(q_dtype, key, ((int64_t)(q0 + t - ctx) * KVH + g) * D + i2);
                        }
                        dot += q * k;
                    }
                    z[t] = dot * (double)scale;
                    if (z[t] > m) m = z[t];
                }
                double l = 0.0;
                for (int t = 0; t < L; ++t) {
                    z[t] = exp(z[t] - m);
                    l += z[t];
                }
                for (int i2 = 0; i2 < D; ++i2) {
                    double acc = 0.0;
                    for (int t = 0; t < L; ++t) {
                        double v;
                        if (t < ctx) {
                            int64_t blk = block_tables[(int64_t)i * max_blocks_per_seq + t / block_size];
                            v = dec(kv_dtype, value_cache, ((blk * KVH + g) * D + i2) * block_size + t % block_size);
                        } else {
                            v = dec(q_dtype, value, ((int64_t)(q0 + t - ctx) * KVH + g) * D + i2);
                        }
                        acc += z[t] * v;
                    }
                    out[((int64_t)(q0 + j) * H + h) * D + i2] = acc / l;
                }
            }
        }
        free(z);
    }
    return 0;
}
