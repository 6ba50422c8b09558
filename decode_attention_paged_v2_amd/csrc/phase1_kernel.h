#pragma once
// Phase 1 of PagedAttention V2 decode on gfx950: one workgroup per
// (sequence, kv head, group of <= 16 query heads, 512-token partition).
//
// What it computes (page "paged_attention_v2_pytorch.py", the per-sequence
// body of paged_attention_v2_pytorch; page "paged_attention_v2_triton.py",
// _paged_attn_v2_partition_kernel for the per-partition decomposition):
// for every query head h of the group and the partition's tokens t,
//   z_t = scale * k_scale * (q_h . K_t) + alibi_h * t,
//   m = max z_t, l = sum exp(z_t - m), o = v_scale * sum exp(z_t - m) V_t / l,
// stored as max_logits, exp_sums and tmp_output.  A partition that starts at
// or past the sequence end only stores max_logits = -inf, exp_sums = 0.
//
// Mapping onto CDNA4:
// * Scores are S^T = K Q^T on 16x16 MFMA tiles: 16 tokens (M) x 16 query
//   heads (N), contracting over the head dimension.  In the key-cache layout
//   [.., d/x, block_size, x] one 16-byte vector is x consecutive head-dim
//   elements of one token, which is exactly one lane's A-operand slice of a
//   16x16x32 (16-bit) step, so K goes from HBM straight into MFMA registers.
// * Tokens are taken 32 at a time as two natural 16-token S^T tiles (K loads
//   stay whole 16-byte vectors of consecutive tokens).  Two cross-lane swaps
//   (v_permlane32_swap, v_permlane16_swap) regroup the scores so each lane
//   holds 8 consecutive tokens of one head: its B-operand slice of a K = 32
//   step of O^T = V^T P^T, whose A-operand slice (the same 8 tokens of one
//   head-dim row) is one contiguous load from the value layout
//   [.., d, block_size]; a lane group's slices cover whole rows.  No LDS
//   traffic sits between the two products.
// * The query heads that share a kv head (GQA) are the N dimension, so each
//   K/V byte is read once per kv head, not once per query head.
// * Two passes per wavefront: all scores of its units first (registers), then
//   one max, then exp and P V with no running rescale.  The wavefronts of a
//   workgroup split the partition's units round-robin and merge their
//   (max, sum, output) once through LDS at the end.
// * K and V loads form one stream of load groups issued a few groups ahead of
//   the MFMAs, so V loads are in flight while the score max is reduced; they
//   carry the non-temporal hint (each byte is read once).
// * P is split into two 16-bit parts (hi + lo) that enter two MFMAs against
//   the same V slice, so the weights keep ~16 significant bits.
// * fp8 e4m3 caches are widened in registers by the hardware converters to
//   the query's 16-bit type (exact) or to f32; k_scale folds into the score
//   scale and v_scale into the final division.
// * exp2 with log2(e) folded into the score scale; ALiBi is added relative to
//   the partition's last token (bias slope * (t - last), |t - last| < 512, so
//   scores stay small where they matter), and the stored max_logits are
//   shifted back to the absolute frame the pages use.
#include <math.h>

#include <atomic>

#include "pav2_internal.h"

namespace pav2 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- 16-bit packing / fp8 widening (gfx950 converters) --------------------

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (DT == BF16) {
        bf16x2 v;
        v[0] = (__bf16)a;
        v[1] = (__bf16)b;
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2 v;
        v[0] = (_Float16)a;
        v[1] = (_Float16)b;
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <int DT>
__device__ __forceinline__ float unpack_lo(uint32_t w) {
    if constexpr (DT == BF16) return as_f32(w << 16);
    else return (float)as_f16x2(w)[0];
}

template <int DT>
__device__ __forceinline__ float unpack_hi(uint32_t w) {
    if constexpr (DT == BF16) return as_f32(w & 0xffff0000u);
    else return (float)as_f16x2(w)[1];
}

// Bytes 0,1 (HI = false) or 2,3 (HI = true) of w, e4m3 -> two 16-bit values.
template <int DT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w) {
    if constexpr (DT == BF16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// ---- MFMA wrappers ----------------------------------------------------------

template <int DT>
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_k4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float wave_sum_groups(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Compile-time shape of one (query dtype, kv dtype, head size) variant.
template <int QDT, int KVDT, int D>
struct Shape {
    static constexpr bool kF32 = (QDT == F32);          // f32 MFMA family
    static constexpr int kKvBytes = KVDT == F32 ? 4 : (KVDT == FP8 ? 1 : 2);
    static constexpr int kX = 16 / kKvBytes;            // elements per 16-byte K vector
    static constexpr int kChunks = D / kX;              // K vectors per token
    static constexpr int kKLoads = (kChunks + 3) / 4;   // K vectors per lane per tile
    static constexpr int kDTiles = (D + 15) / 16;       // 16-row head-dim tiles for P V
    static constexpr int kD16 = kDTiles * 16;
};

template <int N>
struct Words {
    uint32_t w[N];
};

template <typename T>
__device__ __forceinline__ T load_stream(const uint8_t *p) {
    if constexpr (kPhase1NonTemporal)
        return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
    else
        return *reinterpret_cast<const T *>(p);
}

// SCHED: 0 dense grid of partition slots, 1 compact list of used partitions,
// 2 single pass (one workgroup per (sequence, kv head, head group) walks all
// of the sequence's partitions and writes the final output), 3 paged prefix
// attention (the layout kept for f32 queries and head sizes the MFMA prefix
// kernel does not cover), 4 the compact list taken by wavefront items
// (block-sparse only; at most 256 VGPRs, two wavefronts per SIMD).
// BS: the block size when fixed at compile time (16 or 32), 0 for any of
// 8 .. 512, -1 for 1, 2 or 4 (a lane's 8-token V slice then spans blocks).
// SPARSE: the block-sparse pattern of Phase1Params (the dense grid and
// wavefront items): units of a partition that no head of the group attends
// are never loaded, and scores of tokens a head does not attend are masked.
template <int QDT, int KVDT, int D, int WAVES, int SCHED, int BS, bool SPARSE>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(SCHED == 4 ? 2 : kPhase1Occupancy)))
phase1_kernel(const Phase1Params P) {
    // Block-sparse wavefront items: the compact list of used partitions, but
    // each wavefront takes whole items of the workgroup's range by itself
    // (its own table slice, attended units and running softmax, its own
    // outputs; no barrier in the item loop), so that items which attend few
    // units keep four times as many of their latency chains in flight.
    constexpr bool WAVEIT = SCHED == 4;
    static_assert(!WAVEIT || SPARSE, "wavefront items: the block-sparse kernels only");
    constexpr bool COMPACT = SCHED == 1 || WAVEIT;
    // Paged prefix attention: the 16 columns of a group are (query token,
    // head) rows of one chunk, each with its own causal limit, walked like
    // the single pass over the partitions of the sequence.
    constexpr bool PREFIX = SCHED == 3;
    constexpr bool SINGLE = SCHED == 2 || PREFIX;
    using S = Shape<QDT, KVDT, D>;
    constexpr int NKL = S::kKLoads;
    constexpr int NDT = S::kDTiles;
    constexpr int X = S::kX;
    constexpr int KVB = S::kKvBytes;
    constexpr int QB = QDT == F32 ? 4 : 2;            // query element bytes

    extern __shared__ __align__(16) uint8_t smem[];

    const int tid0 = threadIdx.x;

    const int maxP = P.max_num_partitions;
    const int HG = P.head_groups;
    const int KVH = P.num_kv_heads;
    // compact schedule by (kv head, head group) class per XCD (host-checked:
    // KVH * HG is a multiple of 8; the grid, a multiple of 8, is re-checked)
    const bool classes = COMPACT && P.xcd_classes != 0 && (gridDim.x & 7) == 0;
    // (prefix attention merges nothing across wavefronts: no partial-output area)
    const int heads_alloc = PREFIX ? 0 : min(P.gqa, kMaxHeadsPerGroup);
    constexpr int kBsLog2 = BS == 16 ? 4 : (BS == 32 ? 5 : -1);
    const int bs_log2 = kBsLog2 >= 0 ? kBsLog2 : P.bs_log2;
    const int bs_mask = (1 << bs_log2) - 1;
    // LDS: per-wave partial outputs, per-wave max/sums, the partition's
    // block-table slice, then (compact schedule) the partition-count prefix.
    float *s_o = reinterpret_cast<float *>(smem);
    float *s_m = s_o + WAVES * heads_alloc * (S::kD16 + 4);
    float *s_l = s_m + WAVES * kMaxHeadsPerGroup;
    float *s_lr = s_l + WAVES * kMaxHeadsPerGroup;
    int *s_bt = reinterpret_cast<int *>(s_lr + WAVES * kMaxHeadsPerGroup);
    int *s_pref = s_bt + (WAVEIT ? WAVES : 1) * (kPartition >> bs_log2);   // [num_seqs + 1]
    int *s_wsum = s_pref + P.num_seqs + 1;              // [WAVES]
    // block-sparse: each wavefront's bits of the attended-unit mask
    uint32_t *s_umask = reinterpret_cast<uint32_t *>(COMPACT ? s_wsum + WAVES : s_pref);   // [WAVES]

    // Work items.  Dense schedule: one (partition, seq, kv head, head group)
    // slot per workgroup, consecutive slots on one XCD (blockIdx.x % 8).
    // Compact schedule: the workgroup computes the exclusive prefix of the
    // sequences' partition counts from seq_lens in LDS and takes a contiguous
    // range of the list of used (seq, partition, kv head, head group) items;
    // the workgroups of one XCD (blockIdx % 8) take one contiguous block of it.
    // Single pass: the items are the partitions of one (seq, kv head, head
    // group), blockIdx.x, taken in order.
    // Prefix attention: workgroup (sequence, kv head, block of 64 rows), row
    // rr = token j * gqa + head r of the chunk; wavefront w owns rows
    // 16 w .. 16 w + 15 of the block.  All four wavefronts take the same
    // kPrefixSlice-token key slice per item (PAV2_PREFIX_SLICE, a whole
    // 512-token partition by default; each K/V vector is fetched once for 64
    // rows) up to the block's last row's limit context + j + 1, each keeping
    // its rows' running (max, sum, output) in registers.
    int pf_q0 = 0, pf_ctx = 0, pf_rows = 0, pf_lmax = 0;
    // Single pass and prefix: the workgroup's (sequence, kv head, group)
    // index.  Prefix attention numbers its workgroups XCD by XCD (the grid is
    // a multiple of 8, blockIdx % 8 picks the XCD), so the row blocks of one
    // (sequence, kv head), which stream the same keys, share one L2.
    const int wg = PREFIX ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)) : (int)blockIdx.x;
    int item, item_end;
    if constexpr (SINGLE) {
        if (wg >= P.num_work) return;
        int L;
        if constexpr (PREFIX) {
            const int sq = wg / (KVH * HG), rb = wg % HG;
            pf_q0 = P.query_start_loc[sq];
            pf_rows = (P.query_start_loc[sq + 1] - pf_q0) * P.gqa;
            pf_ctx = P.context_lens[sq];
            if (rb * kPrefixRows >= pf_rows) return;   // no rows in this block (uniform)
            pf_lmax = pf_ctx + (min(pf_rows, (rb + 1) * kPrefixRows) - 1) / P.gqa + 1;
            L = pf_lmax;
        } else {
            L = P.seq_lens[wg / (KVH * HG)];
        }
        item = 0;
        const int span = PREFIX ? kPrefixSlice : kPartition;
        item_end = L > 0 ? (L + span - 1) / span : 0;
    } else if constexpr (COMPACT) {
        const int tid = tid0, lane = tid0 & 63, wv = tid0 >> 6;
        const int nthr = WAVES * 64;
        const int per_t = (P.num_seqs + nthr - 1) / nthr;
        auto parts_of = [&](int sq) {
            const int n = (P.seq_lens[sq] + kPartition - 1) / kPartition;
            return n < maxP ? (n > 0 ? n : 0) : maxP;
        };
        int local = 0;
        for (int k = 0; k < per_t; ++k) {
            const int sq = tid * per_t + k;
            if (sq < P.num_seqs) local += parts_of(sq);
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == 63) s_wsum[wv] = incl;
        __syncthreads();
        int run = incl - local, total = 0;
        for (int w2 = 0; w2 < WAVES; ++w2) {
            if (w2 < wv) run += s_wsum[w2];
            total += s_wsum[w2];
        }
        for (int k = 0; k < per_t; ++k) {
            const int sq = tid * per_t + k;
            if (sq < P.num_seqs) {
                s_pref[sq] = run;
                run += parts_of(sq);
            }
        }
        if (tid == 0) s_pref[P.num_seqs] = total;
        total = __builtin_amdgcn_readfirstlane(total);   // wave-uniform: keep the item loop scalar
        __syncthreads();
        if (classes) {
            // XCD x = blockIdx % 8 walks whole (kv head, head group) classes
            // x * C/8 .. (x + 1) * C/8 - 1; items are numbered class-major
            // (class * total + the (sequence, partition) index), and the XCD's
            // workgroups take balanced contiguous ranges of its list
            const int64_t len = (int64_t)total * ((KVH * HG) >> 3);
            const int x = blockIdx.x & 7, bw = blockIdx.x >> 3, nw = gridDim.x >> 3;
            item = (int)(len * x + len * bw / nw);
            item_end = (int)(len * x + len * (bw + 1) / nw);
        } else {
            const int64_t n_items = (int64_t)total * KVH * HG;
            // balanced contiguous ranges; the XCD-blocked numbering is a
            // permutation of the workgroups when the grid is a multiple of 8
            const bool xcd = kPhase1XcdRanges && (gridDim.x & 7) == 0;
            const int b = xcd ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)) : (int)blockIdx.x;
            item = (int)(n_items * b / gridDim.x);
            item_end = (int)(n_items * (b + 1) / gridDim.x);
        }
    } else {
        const int nblk = gridDim.x;
        item = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
        if (item >= P.num_work) return;
        item_end = item + 1;
    }

    // Single pass: the merging threads carry, per output vector they own, the
    // running maximum (log2 units; with ALiBi relative to the last token), the rounded-weight
    // sum and the unnormalised output of the partitions merged so far.
    constexpr int VEC = QDT == F32 ? 4 : 8;
    constexpr int PER_HEAD = D / VEC;
    constexpr int NRUN = (SINGLE && !PREFIX) ? (kMaxHeadsPerGroup * PER_HEAD + WAVES * 64 - 1) / (WAVES * 64) : 1;
    // P V accumulators (O^T tiles), the rounded-weight sums and the exact
    // sums: per item, except in prefix attention, where they run over the
    // whole key range together with the running max pf_m (per column).
    f32x4 o[NDT];
    f32x4 osum = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.0f;
    float pf_m = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float run_m[NRUN], run_l[NRUN], run_o[NRUN][VEC];
#pragma unroll
    for (int k = 0; k < NRUN; ++k) {
        run_m[k] = -INFINITY;
        run_l[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) run_o[k][e] = 0.0f;
    }

    if constexpr (WAVEIT) item += __builtin_amdgcn_readfirstlane(tid0 >> 6);   // wavefront w: items w, w + 4, ...
    for (; item < item_end; item += WAVEIT ? WAVES : 1) {
    int hg = item % HG;
    int s, g, p;
    if constexpr (SINGLE) {
        hg = wg % HG;
        g = (wg / HG) % KVH;
        s = wg / (HG * KVH);
        p = PREFIX ? item / (kPartition / kPrefixSlice) : item;
    } else if constexpr (COMPACT) {
        int r;
        if (classes) {
            const int total = __builtin_amdgcn_readfirstlane(s_pref[P.num_seqs]);
            const int c = item / total;
            r = item - c * total;
            hg = c % HG;
            g = c / HG;
        } else {
            r = item / HG;
            g = r % KVH;
            r /= KVH;
        }
        int lo = 0, hi = P.num_seqs;   // last sequence with prefix <= r (scalar search)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (__builtin_amdgcn_readfirstlane(s_pref[mid]) <= r) lo = mid;
            else hi = mid;
        }
        s = lo;
        p = r - __builtin_amdgcn_readfirstlane(s_pref[lo]);
    } else {
        int w = item / HG;
        g = w % KVH;
        w /= KVH;
        s = w % P.num_seqs;
        p = w / P.num_seqs;
    }
    if constexpr ((COMPACT && !WAVEIT) || SINGLE) __syncthreads();   // the previous item's LDS is free

    // Lane indices.  In the item loop they are taken from an opaque per-item
    // copy of the thread id, so that lane-derived address terms are recomputed
    // per item rather than hoisted out of the loop and kept live across it.
    int tid = tid0;
    if constexpr (COMPACT || SINGLE) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int col = lane & 15;   // token row (K^T loads), head column (outputs), head-dim row (V^T loads)
    const int grp = lane >> 4;   // 4-element slice index within the MFMA operand

    const int L = PREFIX ? pf_lmax : P.seq_lens[s];
    const int start = p * kPartition;
    const int h0 = g * P.gqa + hg * kMaxHeadsPerGroup;
    const int rb0 = (hg * WAVES + wv) * kMaxHeadsPerGroup;   // prefix: this wavefront's first row
    const int nh = PREFIX ? max(0, min(kMaxHeadsPerGroup, pf_rows - rb0))
                          : min(kMaxHeadsPerGroup, P.gqa - hg * kMaxHeadsPerGroup);

    if (start >= L) {   // unused partition slot (dense and compact schedules)
        const int hi = WAVEIT ? lane : tid;
        if (!SINGLE && hi < nh) {
            const int64_t i = ((int64_t)s * P.num_heads + h0 + hi) * maxP + p;
            P.max_logits[i] = -INFINITY;
            P.exp_sums[i] = 0.0f;
        }
        if constexpr (COMPACT || SINGLE) continue;
        else return;
    }
    const int n_tok = min(kPartition, L - start);
    const int last = start + n_tok - 1;   // ALiBi reference position: the partition's last token

    // the partition's block-table slice (wavefront items: each wavefront's own)
    int *const s_btw = WAVEIT ? s_bt + wv * (kPartition >> bs_log2) : s_bt;
    {
        const int n_all = kPartition >> bs_log2;
        const int n_used = (n_tok + bs_mask) >> bs_log2;
        const int32_t *bt = P.block_tables + (int64_t)s * P.max_blocks_per_seq + (start >> bs_log2);
        if constexpr (WAVEIT) {
            for (int i = lane; i < n_all; i += 64) s_btw[i] = i < n_used ? bt[i] : 0;
        } else {
            for (int i = tid; i < n_all; i += WAVES * 64) s_bt[i] = i < n_used ? bt[i] : 0;
        }
    }

    // Query operand (B of S^T = K Q^T): head h0 + col, head-dim slice of K vector
    // (4u + grp), i.e. elements d = X * (4u + grp) + e.
    const bool hvalid = col < nh;
    const uint8_t *qrow;
    int lcol = L;   // prefix attention: this lane's column's causal limit (keys t < lcol)
    if constexpr (PREFIX) {
        const int rr = rb0 + col;
        const int j = rr / P.gqa;
        qrow = reinterpret_cast<const uint8_t *>(P.query) +
               (((int64_t)(pf_q0 + j) * P.num_heads + g * P.gqa + (rr - j * P.gqa)) * D) * QB;
        lcol = hvalid ? pf_ctx + j + 1 : L;
    } else {
        qrow = reinterpret_cast<const uint8_t *>(P.query) + (((int64_t)s * P.num_heads + h0 + col) * D) * QB;
    }
    // the block's smallest column limit (its first row's): units below it need no mask
    const int lmin = PREFIX ? (nh > 0 ? pf_ctx + rb0 / P.gqa + 1 : L) : L;
    Words<X * QB / 4> qw[NKL];
    auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NKL; ++u) {
            const int c = 4 * u + grp;
            const bool ok = hvalid && c < S::kChunks;
#pragma unroll
            for (int k = 0; k < X * QB / 16; ++k) {
                u32x4 v = {0, 0, 0, 0};
                if (ok) v = *reinterpret_cast<const u32x4 *>(qrow + (int64_t)c * X * QB + 16 * k);
                qw[u].w[4 * k + 0] = v[0];
                qw[u].w[4 * k + 1] = v[1];
                qw[u].w[4 * k + 2] = v[2];
                qw[u].w[4 * k + 3] = v[3];
            }
        }
    };
    if constexpr (!WAVEIT) load_q();   // wavefront items load it per chunk

    // ALiBi slope in log2 units (0 without ALiBi, so the bias terms vanish).
    float slope2 = 0.0f;
    if (P.alibi != nullptr && hvalid) slope2 = P.alibi[h0 + col] * kLog2e;
    const float scale_log2 = P.scale_log2;

    // Block-sparse: sparse blocks above sp_klo are the local window; this
    // lane's head attends the stripe residue sp_res (mod vert_stride).  Each
    // thread tests kPartition / (MW * 64) consecutive tokens against every
    // head of the group (MW: the wavefronts sharing the partition), and a
    // ballot gives each wavefront's 32-token units their "attended by some
    // head" bits (wavefront items: all 16 units' bits, in sp_um).
    int sp_res = -1, sp_klo = 0;
    uint32_t sp_um = 0;
    if constexpr (SPARSE) {
        const int vs = P.sp_vert_stride, B = P.sp_block_size;
        sp_klo = (L - 1) / B - P.sp_local_blocks;
        if (hvalid) {
            const int64_t x = (int64_t)(P.tp_rank * P.num_heads + h0 + col) * P.sp_sliding_step;
            const int r = (int)(x % vs);
            sp_res = r < 0 ? r + vs : r;
        }
        int rall[kMaxHeadsPerGroup];   // every head's residue (lane c holds head c's)
#pragma unroll
        for (int c = 0; c < kMaxHeadsPerGroup; ++c) rall[c] = __shfl(sp_res, c);
        constexpr int MW = WAVEIT ? 1 : WAVES;
        constexpr int TPT = kPartition / (MW * 64);   // tokens per thread
        constexpr int TPU = 32 / TPT;                 // threads per 32-token unit
        static_assert(kPartition % (MW * 64) == 0 && TPU >= 1 && TPU <= 64, "unit test layout");
        const int ti = WAVEIT ? lane : tid;
        bool hit = false;
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int t = start + ti * TPT + k;
            if (t < L) {
                const int kb = t / B;
                if (kb > sp_klo) {
                    hit = true;
                } else {
                    const int r = kb % vs;
#pragma unroll
                    for (int c = 0; c < kMaxHeadsPerGroup; ++c) hit = hit || (c < nh && rall[c] == r);
                }
            }
        }
        const uint64_t bal = __ballot(hit);
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < 64 / TPU; ++j)
            if ((bal >> (j * TPU)) & (TPU == 64 ? ~0ull : ((1ull << TPU) - 1))) bits |= 1u << j;
        if constexpr (WAVEIT) sp_um = __builtin_amdgcn_readfirstlane(bits);
        else if (lane == 0) s_umask[wv] = bits << (wv * (64 / TPU));
    }

    if constexpr (WAVEIT) {
        // the wavefront's own slice: its LDS writes precede its reads in
        // program order, and one wavefront's LDS accesses complete in order
        __builtin_amdgcn_wave_barrier();
    } else {
        __syncthreads();   // block-table slice ready (and the attended-unit bits)
    }

    const uint8_t *kc = P.key_cache + (int64_t)g * P.head_stride;
    const uint8_t *vc = P.value_cache + (int64_t)g * P.head_stride;
    const int64_t blk_stride = P.blk_stride;

    // The partition is processed in 32-token units, assigned to the wavefronts
    // round-robin; a unit past the end is clamped to unit 0 (its tokens are
    // then all masked).
    constexpr int UNIT = 32;
    constexpr int UPW = PREFIX ? kPrefixSlice / UNIT : (kPartition / UNIT) / WAVES;   // units per wavefront
    const int nunits = (n_tok + UNIT - 1) / UNIT;
    // Wavefront items walk their attended units UPW at a time (chunks), the
    // running max (pf_m), sums and output carried from chunk to chunk; the
    // other schedules take their units in one pass.
    float m = -INFINITY, lsum_r = 0.0f;
    // (at least one chunk: an item no head attends runs one of unattended entries)
    const int nchunks = WAVEIT ? max(1, (__builtin_popcount(sp_um) + UPW - 1) / UPW) : 1;
    constexpr int RS = S::kD16 + 4;   // row stride (floats) of s_o
    if constexpr (WAVEIT) {
        pf_m = -INFINITY;
        lsum = 0.0f;
        osum = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int ck = 0;
    do {
    if constexpr (WAVEIT) {   // reloaded per chunk, not kept live across one
        asm volatile("" : "+v"(qrow));
        load_q();
    }
    // Block-sparse: the wavefronts deal out the list of attended units
    // (ascending) round-robin (wavefront items: chunk ck of the wavefront's
    // own list); entries past the list's end are -1.  Such an
    // entry still runs the unit's loads and matrix work, but every lane loads
    // the same few lines at the start of the pool (an address select, one
    // line per load instruction), its scores are -inf and its V words
    // zeroed.  Loads thus never depend on a unit's validity: a per-unit
    // condition there costs the kernel about 120 VGPRs, i.e. its second
    // wavefront per SIMD.
    int sp_unit[SPARSE ? UPW : 1];
    if constexpr (WAVEIT) {
        uint32_t um = sp_um;
        for (int i = 0; i < ck * UPW; ++i) um &= um - 1;   // skip the earlier chunks' units
#pragma unroll
        for (int u = 0; u < UPW; ++u) {
            sp_unit[u] = um ? __builtin_ctz(um) : -1;
            um &= um - 1;
        }
    } else if constexpr (SPARSE) {
        uint32_t um = 0;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) um |= s_umask[w2];
        um = __builtin_amdgcn_readfirstlane(um);
        for (int i = 0; i < wv; ++i) um &= um - 1;   // skip the first wv attended units
#pragma unroll
        for (int u = 0; u < UPW; ++u) {
            sp_unit[u] = um ? __builtin_ctz(um) : -1;
            for (int i = 0; i < WAVES; ++i) um &= um - 1;
        }
    }
    auto unit_of = [&](int u) {
        if constexpr (PREFIX) return (item % (kPartition / kPrefixSlice)) * UPW + u;
        else if constexpr (SPARSE) return sp_unit[u] >= 0 ? sp_unit[u] : 0;
        else return wv + WAVES * u;
    };
    auto uvalid = [&](int u) {
        if constexpr (SPARSE) return sp_unit[u] >= 0;
        else return true;
    };
    auto clamp_unit = [&](int t) { return t < nunits ? t : 0; };

    // Load groups: K of a unit in KG groups (halves when large), V of a unit in
    // VSPLIT groups of head-dim tiles; the loads run PF groups ahead of use.
    constexpr int VW = 8 * KVB / 4;                        // words per V slice (8 tokens)
    constexpr int KG = (2 * NKL * 4 > 32) ? 2 : 1;
    constexpr int KH = 2 / KG;                             // K halves per group
    constexpr int VSPLIT = (NDT * VW > 32) ? 2 : 1;
    constexpr int DPG = (NDT + VSPLIT - 1) / VSPLIT;       // head-dim tiles per V group
    constexpr int GK = UPW * KG;
    constexpr int NG = GK + UPW * VSPLIT;
    constexpr int PF = (KH * NKL * 4 <= 16 && DPG * VW <= 16) ? 3 : 2;

    // ---- load helpers ----------------------------------------------------
    auto load_k = [&](u32x4 (&dst)[NKL], int u, int half) {
        const int t = clamp_unit(unit_of(u));
        const int o = t * UNIT + 16 * half + col;            // token offset in partition
        const uint8_t *base;
        if constexpr (BS >= 16) {
            // the tile's 16 tokens share one block: a wave-uniform block base
            // plus a per-lane offset that does not change between tiles
            const int64_t b = __builtin_amdgcn_readfirstlane(s_btw[(t * UNIT + 16 * half) >> bs_log2]);
            const uint32_t lane_off = (uint32_t)((o & bs_mask) * 16 + (grp << (bs_log2 + 4)));
            base = kc + b * blk_stride + lane_off;
        } else {
            const int64_t b = s_btw[o >> bs_log2];
            base = kc + b * blk_stride + (o & bs_mask) * 16 + (grp << (bs_log2 + 4));
        }
        if constexpr (SPARSE) base = uvalid(u) ? base : kc;
#pragma unroll
        for (int w = 0; w < NKL; ++w) {
            u32x4 v = {0, 0, 0, 0};
            if (4 * w + grp < S::kChunks)
                v = load_stream<u32x4>(base + ((int64_t)(4 * w) << (bs_log2 + 4)));
            dst[w] = v;
        }
    };
    auto load_v = [&](Words<VW> (&dst)[DPG], int u, int part) {
        const int t = clamp_unit(unit_of(u));
        const int o = t * UNIT + 8 * grp;                    // first of the lane's 8 tokens
        if constexpr (BS < 0) {
            // blocks of 1, 2 or 4 tokens: the lane's 8 tokens span 8 / block_size
            // blocks, so each token's element comes from its own block's row
            const uint8_t *tb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tok = o + e;
                tb[e] = vc + (int64_t)s_btw[tok >> bs_log2] * blk_stride + ((tok & bs_mask) + (col << bs_log2)) * KVB;
                if constexpr (SPARSE) tb[e] = uvalid(u) ? tb[e] : vc;
            }
#pragma unroll
            for (int i = 0; i < DPG; ++i) {
                const int dt = part * DPG + i;
                if (dt >= NDT) break;
                const bool ok = (D % 16 == 0) || (16 * dt + col < D);
                const int64_t roff = ((int64_t)(16 * dt) << bs_log2) * KVB;
                uint32_t el[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t v = 0u;
                    if (ok) {
                        if constexpr (KVB == 4) v = *reinterpret_cast<const uint32_t *>(tb[e] + roff);
                        else if constexpr (KVB == 2) v = *reinterpret_cast<const uint16_t *>(tb[e] + roff);
                        else v = *(tb[e] + roff);
                    }
                    el[e] = v;
                }
#pragma unroll
                for (int w = 0; w < VW; ++w) {
                    if constexpr (KVB == 4) dst[i].w[w] = el[w];
                    else if constexpr (KVB == 2) dst[i].w[w] = el[2 * w] | (el[2 * w + 1] << 16);
                    else dst[i].w[w] = el[4 * w] | (el[4 * w + 1] << 8) | (el[4 * w + 2] << 16) | (el[4 * w + 3] << 24);
                }
            }
        } else {
        const uint8_t *base;
        if constexpr (BS >= 32) {
            // the unit's 32 tokens share one block
            const int64_t b = __builtin_amdgcn_readfirstlane(s_btw[(t * UNIT) >> bs_log2]);
            const uint32_t lane_off = (uint32_t)(((o & bs_mask) + (col << bs_log2)) * KVB);
            base = vc + b * blk_stride + lane_off;
        } else {
            const int64_t b = s_btw[o >> bs_log2];
            base = vc + b * blk_stride + (o & bs_mask) * KVB + (col << bs_log2) * KVB;
        }
        if constexpr (SPARSE) base = uvalid(u) ? base : vc;
#pragma unroll
        for (int i = 0; i < DPG; ++i) {
            const int dt = part * DPG + i;
            if (dt >= NDT) break;
            const uint8_t *ptr = base + ((int64_t)(16 * dt) << bs_log2) * KVB;
            const bool ok = (D % 16 == 0) || (16 * dt + col < D);
            if constexpr (VW == 2) {
                u32x2 v = {0, 0};
                if (ok) v = load_stream<u32x2>(ptr);
                dst[i].w[0] = v[0];
                dst[i].w[1] = v[1];
            } else {
#pragma unroll
                for (int h = 0; h < VW / 4; ++h) {
                    u32x4 v = {0, 0, 0, 0};
                    if (ok) v = load_stream<u32x4>(ptr + 16 * h);
                    dst[i].w[4 * h + 0] = v[0];
                    dst[i].w[4 * h + 1] = v[1];
                    dst[i].w[4 * h + 2] = v[2];
                    dst[i].w[4 * h + 3] = v[3];
                }
            }
        }
        }
    };

    // ---- S^T tile from K vectors ---------------------------------------------
    auto qk_tile = [&](const u32x4 (&kr)[NKL]) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NKL; ++u) {
            if constexpr (!S::kF32 && KVDT != FP8) {
                u32x4 qv = {qw[u].w[0], qw[u].w[1], qw[u].w[2], qw[u].w[3]};
                acc = mfma_k32<QDT>(kr[u], qv, acc);
            } else if constexpr (!S::kF32) {   // fp8 K -> 16-bit, two steps per vector
                u32x4 k0 = {fp8x2_to_16<QDT, false>(kr[u][0]), fp8x2_to_16<QDT, true>(kr[u][0]),
                            fp8x2_to_16<QDT, false>(kr[u][1]), fp8x2_to_16<QDT, true>(kr[u][1])};
                u32x4 k1 = {fp8x2_to_16<QDT, false>(kr[u][2]), fp8x2_to_16<QDT, true>(kr[u][2]),
                            fp8x2_to_16<QDT, false>(kr[u][3]), fp8x2_to_16<QDT, true>(kr[u][3])};
                u32x4 q0 = {qw[u].w[0], qw[u].w[1], qw[u].w[2], qw[u].w[3]};
                u32x4 q1 = {qw[u].w[4], qw[u].w[5], qw[u].w[6], qw[u].w[7]};
                acc = mfma_k32<QDT>(k0, q0, acc);
                acc = mfma_k32<QDT>(k1, q1, acc);
            } else if constexpr (KVDT == F32) {   // f32: four 16x16x4 steps per vector
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma_k4(as_f32(kr[u][e]), as_f32(qw[u].w[e]), acc);
            } else {                              // fp8 K with f32 query
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    f32x2 lo = fp8x2_to_f32<false>(kr[u][wd]);
                    f32x2 hi = fp8x2_to_f32<true>(kr[u][wd]);
                    acc = mfma_k4(lo[0], as_f32(qw[u].w[4 * wd + 0]), acc);
                    acc = mfma_k4(lo[1], as_f32(qw[u].w[4 * wd + 1]), acc);
                    acc = mfma_k4(hi[0], as_f32(qw[u].w[4 * wd + 2]), acc);
                    acc = mfma_k4(hi[1], as_f32(qw[u].w[4 * wd + 3]), acc);
                }
            }
        }
        return acc;
    };

    if constexpr (!PREFIX && !WAVEIT) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    u32x4 kbuf[PF][KH][NKL];
    Words<VW> vbuf[PF][DPG];
    float sc[UPW][8];                 // scores of the lane's 8 tokens per unit (log2 units)

    auto issue = [&](int j) {
        if (j < GK) {
#pragma unroll
            for (int hh = 0; hh < KH; ++hh) load_k(kbuf[j % PF][hh], j / KG, (j % KG) * KH + hh);
        } else if (j < NG) {
            load_v(vbuf[j % PF], (j - GK) / VSPLIT, (j - GK) % VSPLIT);
        }
    };

#pragma unroll
    for (int j = 0; j < PF; ++j) issue(j);

    // Pass 1: scores of every unit.  Tile `half` of a unit holds tokens
    // 16 * half + 4 * grp + i in the lane's accumulator element i.
#pragma unroll
    for (int j = 0; j < GK; ++j) {
        const int u = j / KG;
        f32x4 acc[KH];
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) acc[hh] = qk_tile(kbuf[j % PF][hh]);
        issue(j + PF);
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) {
            const int half = (j % KG) * KH + hh;
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[u][4 * half + i] = acc[hh][i];
        }
    }
    // Regroup each unit's scores so that lane group g holds tokens 8g .. 8g+7:
    // swapping the upper 32 lanes of the first tile with the lower 32 of the
    // second, then odd 16-lane rows of the first with even rows of the second,
    // leaves tokens 8g + i in the first register and 8g + 4 + i in the second.
    // Then scale and ALiBi bias (slope * (t - last), the lane's first token of
    // unit u being t = start + (wv + WAVES u) * 32 + 8 grp); tokens at or past
    // the sequence end (only in the last unit, or in a clamped one) get -inf.
    const float bias0 = slope2 * (float)(start + wv * UNIT + 8 * grp - last);
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane32_swap(as_u32(sc[u][i]), as_u32(sc[u][4 + i]), false, false);
            const auto q = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
            sc[u][i] = as_f32(q[0]);
            sc[u][4 + i] = as_f32(q[1]);
        }
        float bu = u == 0 ? bias0 : fmaf(slope2, (float)(WAVES * UNIT * u), bias0);
        if constexpr (SPARSE) bu = slope2 * (float)(start + unit_of(u) * UNIT + 8 * grp - last);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sc[u][e] = fmaf(sc[u][e], scale_log2, e == 0 ? bu : fmaf(slope2, (float)e, bu));
        const int tu = start + unit_of(u) * UNIT;   // unclamped first token of the unit
        if (tu + UNIT > lmin) {
            const int nv = lcol - (tu + 8 * grp);   // valid tokens among the lane's 8
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[u][e] = e < nv ? sc[u][e] : -INFINITY;
        }
        if constexpr (SPARSE) {
            const int B = P.sp_block_size, vs = P.sp_vert_stride;
            if (!uvalid(u)) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sc[u][e] = -INFINITY;
            } else if (tu / B <= sp_klo) {   // not wholly inside the local window: test each token
                const int t0 = tu + 8 * grp;
                int kb = t0 / B, nb = (kb + 1) * B, r = kb % vs;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (t0 + e >= nb) {   // next sparse block (B >= 1: at most one step per token)
                        ++kb;
                        nb += B;
                        r = r + 1 == vs ? 0 : r + 1;
                    }
                    sc[u][e] = (kb > sp_klo || r == sp_res) ? sc[u][e] : -INFINITY;
                }
            }
        }
    }

    m = -INFINITY;
#pragma unroll
    for (int u = 0; u < UPW; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, sc[u][e]);
    m = wave_max(m);
    float mu = (m == -INFINITY) ? 0.0f : m;
    if constexpr (WAVEIT) {   // the running output: zero, or the earlier chunks' from the wavefront's LDS rows
        const float *src = s_o + (wv * heads_alloc + col) * RS;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int row = 16 * dt + 4 * grp;
            o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ck > 0 && hvalid && row < D) o[dt] = *reinterpret_cast<const f32x4 *>(src + row);
        }
    }
    if constexpr (PREFIX || WAVEIT) {   // rescale the running state to the new running max
        const float mn = fmaxf(pf_m, m);
        const float fo = mn == -INFINITY ? 1.0f : exp2_fast(pf_m - mn);
        pf_m = mn;
        mu = mn == -INFINITY ? 0.0f : mn;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[dt][i] *= fo;
#pragma unroll
        for (int i = 0; i < 4; ++i) osum[i] *= fo;
        lsum *= fo;
    }

    // Pass 2: exp and P V.  lsum is the exact sum of the weights (stored as
    // exp_sums); lsum_r sums the weights as they enter the MFMAs, so that the
    // partition output is a true weighted mean of V rows.  16-bit operands
    // carry P as hi + lo, two 16-bit parts (~16 significant bits).
    // The rounded weights' sum comes from one more MFMA pair per unit against
    // an all-ones A operand (every row of that tile is sum_t P[t][head]).
    lsum_r = 0.0f;
    if constexpr (!PREFIX && !WAVEIT) lsum = 0.0f;
    float pr[8];
    u32x4 ph = {0u, 0u, 0u, 0u}, pl = {0u, 0u, 0u, 0u};
    if constexpr (!PREFIX && !WAVEIT) osum = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = pack2<QDT == F32 ? BF16 : QDT>(1.0f, 1.0f);
    const u32x4 ones = {one2, one2, one2, one2};
    // Raw-word masks zeroing V of tokens past the sequence end (word w of a
    // lane's 8-token slice holds tokens w * TPW .. w * TPW + TPW - 1).
    constexpr int TPW = 4 / KVB;
    uint32_t vmask[VW];
    bool vpartial = false;
#pragma unroll
    for (int j = GK; j < NG; ++j) {
        const int u = (j - GK) / VSPLIT;
        const int part = (j - GK) % VSPLIT;
        if (part == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pr[e] = exp2_fast(sc[u][e] - mu);
                lsum += pr[e];
            }
            if constexpr (!S::kF32) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t h = pack2<QDT>(pr[2 * k], pr[2 * k + 1]);
                    const float r0 = pr[2 * k] - unpack_lo<QDT>(h);
                    const float r1 = pr[2 * k + 1] - unpack_hi<QDT>(h);
                    ph[k] = h;
                    pl[k] = pack2<QDT>(r0, r1);
                }
                osum = mfma_k32<QDT>(ones, ph, osum);
                osum = mfma_k32<QDT>(ones, pl, osum);
            }
            const int tu = start + unit_of(u) * UNIT;
            bool unattended = false;   // block-sparse: an entry past the attended list: V words zeroed
            if constexpr (SPARSE) unattended = !uvalid(u);
            vpartial = unattended || tu + UNIT > L;
            if (vpartial) {
                const int nv = unattended ? 0 : L - (tu + 8 * grp);
#pragma unroll
                for (int w = 0; w < VW; ++w) {
                    const int nb = min(max(nv - w * TPW, 0), TPW) * KVB;   // valid bytes of the word
                    vmask[w] = nb >= 4 ? ~0u : (1u << (8 * nb)) - 1u;
                }
            }
        }
        Words<VW> (&vr)[DPG] = vbuf[j % PF];
        if (vpartial) {
#pragma unroll
            for (int i = 0; i < DPG; ++i) {
                if (part * DPG + i >= NDT) break;
#pragma unroll
                for (int w = 0; w < VW; ++w) vr[i].w[w] &= vmask[w];
            }
        }
#pragma unroll
        for (int i = 0; i < DPG; ++i) {
            const int dt = part * DPG + i;
            if (dt >= NDT) break;
            if constexpr (!S::kF32) {
                u32x4 a;
                if constexpr (KVDT == FP8) {
                    a[0] = fp8x2_to_16<QDT, false>(vr[i].w[0]);
                    a[1] = fp8x2_to_16<QDT, true>(vr[i].w[0]);
                    a[2] = fp8x2_to_16<QDT, false>(vr[i].w[1]);
                    a[3] = fp8x2_to_16<QDT, true>(vr[i].w[1]);
                } else {
                    a = u32x4{vr[i].w[0], vr[i].w[1], vr[i].w[2], vr[i].w[3]};
                }
                o[dt] = mfma_k32<QDT>(a, ph, o[dt]);
                o[dt] = mfma_k32<QDT>(a, pl, o[dt]);
            } else {
                float a[8];
                if constexpr (KVDT == FP8) {
#pragma unroll
                    for (int wd = 0; wd < 2; ++wd) {
                        f32x2 lo = fp8x2_to_f32<false>(vr[i].w[wd]);
                        f32x2 hi = fp8x2_to_f32<true>(vr[i].w[wd]);
                        a[4 * wd + 0] = lo[0];
                        a[4 * wd + 1] = lo[1];
                        a[4 * wd + 2] = hi[0];
                        a[4 * wd + 3] = hi[1];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = as_f32(vr[i].w[e]);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) o[dt] = mfma_k4(a[e], pr[e], o[dt]);
            }
        }
        issue(j + PF);
    }
    if constexpr (WAVEIT) {   // more chunks to come: park the running output in the wavefront's LDS rows
        if (ck + 1 < nchunks && hvalid) {
            float *dst = s_o + (wv * heads_alloc + col) * RS;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int row = 16 * dt + 4 * grp;
                if (row < D) *reinterpret_cast<f32x4 *>(dst + row) = o[dt];
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    } while (++ck < nchunks);   // chunks
    if constexpr (WAVEIT) {
        // the wavefront's own partition: statistics and normalised rows, in
        // the merge's format (a head that attends nothing: -inf / 0 and a
        // zero row)
        lsum = wave_sum_groups(lsum);
        const float lr = S::kF32 ? lsum : osum[0];
        if (hvalid) {
            const int64_t srow = (int64_t)s * P.num_heads + h0 + col;
            const float inv = lr > 0.0f ? P.v_scale / lr : 0.0f;
            uint8_t *base = reinterpret_cast<uint8_t *>(P.tmp_out) + (srow * maxP + p) * D * QB;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int d0 = 16 * dt + 4 * grp;   // this lane's 4 consecutive head-dim elements
                if (d0 < D) {
                    const float r0 = o[dt][0] * inv, r1 = o[dt][1] * inv, r2 = o[dt][2] * inv, r3 = o[dt][3] * inv;
                    if constexpr (QDT == F32)
                        *reinterpret_cast<f32x4 *>(base + d0 * QB) = f32x4{r0, r1, r2, r3};
                    else
                        *reinterpret_cast<u32x2 *>(base + d0 * QB) = u32x2{pack2<QDT>(r0, r1), pack2<QDT>(r2, r3)};
                }
            }
            if (grp == 0) {
                float mabs = pf_m * kLn2;
                if (P.alibi != nullptr) mabs += P.alibi[h0 + col] * (float)last;
                P.max_logits[srow * maxP + p] = mabs;
                P.exp_sums[srow * maxP + p] = lsum;
            }
        }
        continue;
    }
    if constexpr (PREFIX) continue;   // the running state stays in registers
    lsum = wave_sum_groups(lsum);
    if constexpr (S::kF32) lsum_r = lsum;
    else lsum_r = osum[0];

    // ---- merge the wavefronts through LDS ---------------------------------------
    if (hvalid) {
        if (grp == 0) {
            s_m[wv * kMaxHeadsPerGroup + col] = m;
            s_l[wv * kMaxHeadsPerGroup + col] = lsum;
            s_lr[wv * kMaxHeadsPerGroup + col] = lsum_r;
        }
        float *dst = s_o + (wv * heads_alloc + col) * RS;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int row = 16 * dt + 4 * grp;
            if (row < D) *reinterpret_cast<f32x4 *>(dst + row) = o[dt];
        }
    }
    __syncthreads();

    const float v_scale = P.v_scale;
    // The wavefronts' (max, sums, unnormalised output) of one output vector,
    // brought to the largest wavefront maximum.
    auto combine = [&](int hh, int d0, float &M, float &l, float &lr, float (&a)[VEC]) {
        M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) M = fmaxf(M, s_m[w2 * kMaxHeadsPerGroup + hh]);
        float f[WAVES];
        l = 0.0f;
        lr = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) {
            const float mw = s_m[w2 * kMaxHeadsPerGroup + hh];
            f[w2] = mw == -INFINITY ? 0.0f : exp2_fast(mw - M);
            l += f[w2] * s_l[w2 * kMaxHeadsPerGroup + hh];
            lr += f[w2] * s_lr[w2 * kMaxHeadsPerGroup + hh];
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < WAVES; ++w2) acc += f[w2] * s_o[(w2 * heads_alloc + hh) * RS + d0 + e];
            a[e] = acc;
        }
    };
    if constexpr (SINGLE) {
        // fold this partition into the running state, rescaling whichever
        // side has the smaller maximum
#pragma unroll
        for (int k = 0; k < NRUN; ++k) {
            const int idx = tid + k * WAVES * 64;
            if (idx < nh * PER_HEAD) {
                const int hh = idx / PER_HEAD;
                const int d0 = (idx - hh * PER_HEAD) * VEC;
                float M, l, lr, a[VEC];
                combine(hh, d0, M, l, lr, a);
                // ALiBi: partition maxima are relative to the partition's last
                // token; the running merge takes them relative to the
                // sequence's last token (nothing is stored, so any per-head
                // frame serves), where the partitions that carry weight have
                // small maxima and float32 resolves their differences finely
                if (!PREFIX && P.alibi != nullptr) M += P.alibi[h0 + hh] * kLog2e * (float)(last - (L - 1));
                const float Mn = fmaxf(run_m[k], M);
                const float fo = exp2_fast(run_m[k] - Mn);   // 0 for the first partition
                const float fn = exp2_fast(M - Mn);
                run_m[k] = Mn;
                run_l[k] = run_l[k] * fo + lr * fn;
#pragma unroll
                for (int e = 0; e < VEC; ++e) run_o[k][e] = run_o[k][e] * fo + a[e] * fn;
            }
        }
        continue;
    }
    for (int idx = tid; idx < nh * PER_HEAD; idx += WAVES * 64) {
        const int hh = idx / PER_HEAD;
        const int d0 = (idx - hh * PER_HEAD) * VEC;
        float M, l, lr, r[VEC];
        combine(hh, d0, M, l, lr, r);
        // block-sparse: a head may attend no token of the partition (l = 0):
        // its row is zero and its statistics -inf / 0, weight 0 in phase 2
        const float inv = SPARSE ? (lr > 0.0f ? v_scale / lr : 0.0f) : v_scale / lr;
#pragma unroll
        for (int e = 0; e < VEC; ++e) r[e] *= inv;
        const int h = h0 + hh;
        const int64_t srow = (int64_t)s * P.num_heads + h;
        uint8_t *dst = reinterpret_cast<uint8_t *>(P.tmp_out) + ((srow * maxP + p) * D + d0) * QB;
        if constexpr (QDT == F32) {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{r[0], r[1], r[2], r[3]};
        } else {
            u32x4 pk = {pack2<QDT>(r[0], r[1]), pack2<QDT>(r[2], r[3]), pack2<QDT>(r[4], r[5]),
                        pack2<QDT>(r[6], r[7])};
            *reinterpret_cast<u32x4 *>(dst) = pk;
        }
        if (d0 == 0) {
            float mabs = M * kLn2;
            if (P.alibi != nullptr) mabs += P.alibi[h] * (float)last;
            P.max_logits[srow * maxP + p] = mabs;
            P.exp_sums[srow * maxP + p] = l;
        }
    }
        if constexpr (!COMPACT) break;
    }   // item loop

    if constexpr (PREFIX) {   // each wavefront normalises and writes its own 16 rows
        const int lane = tid0 & 63, wv = __builtin_amdgcn_readfirstlane(tid0 >> 6);
        const int col = lane & 15, grp = lane >> 4;
        const int hg = wg % HG, g = (wg / HG) % KVH;
        const int rb0 = (hg * WAVES + wv) * kMaxHeadsPerGroup;
        float lr;
        if constexpr (S::kF32) lr = wave_sum_groups(lsum);
        else lr = osum[0];
        if (col < pf_rows - rb0) {
            const int rr = rb0 + col, j = rr / P.gqa;
            const int64_t orow = (int64_t)(pf_q0 + j) * P.num_heads + g * P.gqa + (rr - j * P.gqa);
            const float inv = lr > 0.0f ? P.v_scale / lr : 0.0f;
            uint8_t *base = reinterpret_cast<uint8_t *>(P.tmp_out) + orow * D * QB;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int d0 = 16 * dt + 4 * grp;   // this lane's 4 consecutive head-dim elements
                if (d0 < D) {
                    const float r0 = o[dt][0] * inv, r1 = o[dt][1] * inv, r2 = o[dt][2] * inv, r3 = o[dt][3] * inv;
                    if constexpr (QDT == F32)
                        *reinterpret_cast<f32x4 *>(base + d0 * QB) = f32x4{r0, r1, r2, r3};
                    else
                        *reinterpret_cast<u32x2 *>(base + d0 * QB) = u32x2{pack2<QDT>(r0, r1), pack2<QDT>(r2, r3)};
                }
            }
        }
        return;
    }
    if constexpr (SINGLE) {   // the normalised output, written once (zero rows for an empty sequence)
        const int hg = wg % HG, g = (wg / HG) % KVH, s = wg / (HG * KVH);
        const int h0 = g * P.gqa + hg * kMaxHeadsPerGroup;
        const int nh = min(kMaxHeadsPerGroup, P.gqa - hg * kMaxHeadsPerGroup);
#pragma unroll
        for (int k = 0; k < NRUN; ++k) {
            const int idx = tid0 + k * WAVES * 64;
            if (idx < nh * PER_HEAD) {
                const int hh = idx / PER_HEAD;
                const int d0 = (idx - hh * PER_HEAD) * VEC;
                const float inv = run_l[k] > 0.0f ? P.v_scale / run_l[k] : 0.0f;
                float r[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) r[e] = run_o[k][e] * inv;
                const int64_t orow = (int64_t)s * P.num_heads + h0 + hh;   // output row (sequence, head)
                uint8_t *dst = reinterpret_cast<uint8_t *>(P.tmp_out) + (orow * D + d0) * QB;
                if constexpr (QDT == F32) {
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{r[0], r[1], r[2], r[3]};
                } else {
                    u32x4 pk = {pack2<QDT>(r[0], r[1]), pack2<QDT>(r[2], r[3]), pack2<QDT>(r[4], r[5]),
                                pack2<QDT>(r[6], r[7])};
                    *reinterpret_cast<u32x4 *>(dst) = pk;
                }
            }
        }
    }

    if constexpr (COMPACT) {   // unused slots p >= P_s of this workgroup's share of sequences
        for (int sq = blockIdx.x; sq < P.num_seqs; sq += gridDim.x) {
            const int used = s_pref[sq + 1] - s_pref[sq];
            const int spare = maxP - used;
            const int n = P.num_heads * spare;
            for (int idx = tid0; idx < n; idx += WAVES * 64) {
                const int h = idx / spare;
                const int64_t i = ((int64_t)sq * P.num_heads + h) * maxP + used + (idx - h * spare);
                P.max_logits[i] = -INFINITY;
                P.exp_sums[i] = 0.0f;
            }
        }
    }
}

constexpr int kMaxDevices = 64;

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

int device_cu_count(int dev) {
    static std::atomic<int> cache[kMaxDevices];
    if (dev < 0) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Host state of one kernel variant, per device: the largest dynamic LDS size
// it has been allowed, and its resident workgroups per CU at the last LDS
// size asked for (packed (lds << 32) | workgroups in one atomic word), so a
// launch queries the runtime only when the LDS size changes.
struct VariantState {
    std::atomic<int> lds_allowed[kMaxDevices];
    std::atomic<uint64_t> occupancy[kMaxDevices];
};

hipError_t allow_lds(VariantState &st, const void *fn, int dev, int lds) {
    if (lds <= 65536) return hipSuccess;
    if (dev >= 0 && st.lds_allowed[dev].load(std::memory_order_relaxed) >= lds) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && dev >= 0) st.lds_allowed[dev].store(lds, std::memory_order_relaxed);
    return e;
}

int resident_per_cu(VariantState &st, const void *fn, int dev, int threads, int lds) {
    if (dev >= 0) {
        const uint64_t c = st.occupancy[dev].load(std::memory_order_relaxed);
        if (c != 0 && (int)(c >> 32) == lds) return (int)(c & 0xffffffffu);
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    if (dev >= 0) st.occupancy[dev].store(((uint64_t)(uint32_t)lds << 32) | (uint32_t)per_cu, std::memory_order_relaxed);
    return per_cu;
}

template <int QDT, int KVDT, int D, int SCHED, int BS, bool SPARSE>
hipError_t launch_sched(const Phase1Params &p, int lds, hipStream_t stream) {
    constexpr int WAVES = kPhase1Waves;
    static VariantState state;
    const void *fn = reinterpret_cast<const void *>(&phase1_kernel<QDT, KVDT, D, WAVES, SCHED, BS, SPARSE>);
    const int dev = current_device();
    const hipError_t e = allow_lds(state, fn, dev, lds);
    if (e != hipSuccess) return e;
    int grid = (p.num_work + 7) / 8 * 8;
    if (SCHED == 1 || SCHED == 4) {
        // at most p.compact_rounds resident rounds of workgroups (wavefront
        // items: one round, each workgroup's range shared by its four
        // wavefronts), each walking a balanced range of the used items
        const int rounds = SCHED == 4 ? 1 : p.compact_rounds;
        const int cap = rounds * device_cu_count(dev) * resident_per_cu(state, fn, dev, WAVES * 64, lds);
        grid = grid < cap ? grid : cap;
    } else if (SCHED == 2) {
        grid = p.num_work;   // one workgroup per (sequence, kv head, head group)
    } else if (SCHED == 3) {
        grid = (p.num_work + 7) / 8 * 8;   // one per (sequence, kv head, row block), a multiple of 8
    }
    hipLaunchKernelGGL((phase1_kernel<QDT, KVDT, D, WAVES, SCHED, BS, SPARSE>), dim3(grid), dim3(WAVES * 64), lds,
                       stream, p);
    return hipGetLastError();
}

// Block sizes 16 and 32 (16-bit queries) get kernels with the block size
// fixed at compile time (load offsets become immediates; the block of a
// 16-token K tile, and at 32 of a whole unit, is wave-uniform); blocks of 1,
// 2 or 4 tokens a kernel whose V gather takes each token from its own block
// (BS = -1); every other case runs the generic kernel.
template <int QDT, int KVDT, int D, int SCHED, bool SPARSE>
hipError_t launch_bs(const Phase1Params &p, int lds, hipStream_t stream) {
    if (p.bs_log2 < 3) return launch_sched<QDT, KVDT, D, SCHED, -1, SPARSE>(p, lds, stream);   // blocks of 1, 2, 4
    if constexpr (QDT != F32 && !SPARSE) {
        if (p.bs_log2 == 4) return launch_sched<QDT, KVDT, D, SCHED, 16, false>(p, lds, stream);
        if (p.bs_log2 == 5) return launch_sched<QDT, KVDT, D, SCHED, 32, false>(p, lds, stream);
    }
    return launch_sched<QDT, KVDT, D, SCHED, 0, SPARSE>(p, lds, stream);
}

template <int QDT, int KVDT, int D, bool SPARSE>
hipError_t launch_one(const Phase1Params &p, int lds, hipStream_t stream) {
    if constexpr (SPARSE) {   // block-sparse: the dense grid, or the compact list taken by wavefront items
        switch (p.sched) {
        case 0: return launch_bs<QDT, KVDT, D, 0, true>(p, lds, stream);
        case 1: return launch_bs<QDT, KVDT, D, 4, true>(p, lds, stream);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.sched) {
        case 0: return launch_bs<QDT, KVDT, D, 0, false>(p, lds, stream);
        case 1: return launch_bs<QDT, KVDT, D, 1, false>(p, lds, stream);
        case 2: return launch_bs<QDT, KVDT, D, 2, false>(p, lds, stream);
        case 3:
            if constexpr (QDT == KVDT) return launch_bs<QDT, KVDT, D, 3, false>(p, lds, stream);   // 16/32-bit caches
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
        }
    }
}

template <int QDT, int KVDT, bool SPARSE>
hipError_t launch_d(const Phase1Params &p, int D, int lds, hipStream_t stream) {
    switch (D) {
    case 64: return launch_one<QDT, KVDT, 64, SPARSE>(p, lds, stream);
    case 80: return launch_one<QDT, KVDT, 80, SPARSE>(p, lds, stream);
    case 96: return launch_one<QDT, KVDT, 96, SPARSE>(p, lds, stream);
    case 112: return launch_one<QDT, KVDT, 112, SPARSE>(p, lds, stream);
    case 128: return launch_one<QDT, KVDT, 128, SPARSE>(p, lds, stream);
    case 192: return launch_one<QDT, KVDT, 192, SPARSE>(p, lds, stream);
    case 256: return launch_one<QDT, KVDT, 256, SPARSE>(p, lds, stream);
    case 120:
        if constexpr (KVDT != FP8) return launch_one<QDT, KVDT, 120, SPARSE>(p, lds, stream);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace pav2
