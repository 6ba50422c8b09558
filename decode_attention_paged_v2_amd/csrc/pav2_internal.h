// Internal declarations shared by the PagedAttention V2 kernels and the C ABI.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA 16x16xK tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pav2 {

constexpr int kPartition = 512;                 // tokens per partition
constexpr int kMaxHeadsPerGroup = 16;           // query heads per MFMA N-tile
constexpr int kMaxPartitions = 16384;

enum Dtype { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Scalar reinterpretation goes through these by-value helpers: with this
// compiler, __builtin_bit_cast applied directly to an element of an
// ext_vector_type lvalue (v[i]) reinterprets the vector's first element
// whatever i is, so elements are always copied out as values first.
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }

struct Phase1Params {
    void *tmp_out;                 // [S, H, maxP, D] out dtype; single pass: the output [S, H, D]
    float *exp_sums;               // [S, H, maxP]
    float *max_logits;             // [S, H, maxP]
    const void *query;             // [S, H, D]
    const uint8_t *key_cache;      // [NB, KVH, D/x, BS, x]
    const uint8_t *value_cache;    // [NB, KVH, D, BS]
    const int32_t *block_tables;   // [S, MBPS]
    const int32_t *seq_lens;       // [S]
    const float *alibi;            // [H] or null
    const int32_t *query_start_loc;  // prefix attention: [S + 1] first query row of each chunk
    const int32_t *context_lens;     // prefix attention: [S] tokens before each chunk
    int num_seqs, num_heads, num_kv_heads;
    int gqa;                       // num_heads / num_kv_heads
    int head_groups;               // ceil(gqa / 16)
    int bs_log2;                   // log2(block_size)
    int max_blocks_per_seq;
    int max_num_partitions;
    int num_work;                  // S * KVH * head_groups * maxP (single pass: without maxP)
    int sched;                     // 0 dense slots, 1 compact list of used partitions, 2 single pass,
                                   // 3 prefix attention (head_groups = blocks of kPrefixRows rows)
    int64_t blk_stride;            // bytes per physical block (all kv heads)
    int64_t head_stride;           // bytes per (block, kv head)
    float scale_log2;              // scale * k_scale * log2(e)
    float v_scale;
    // block-sparse pattern (sp_vert_stride > 1; the dense kernels ignore it):
    // head h (model-wide index tp_rank * num_heads + h) attends token t when
    // t / sp_block_size > (L - 1) / sp_block_size - sp_local_blocks or
    // (t / sp_block_size - h' * sp_sliding_step) mod sp_vert_stride == 0
    int tp_rank = 0, sp_local_blocks = 0, sp_vert_stride = 0, sp_block_size = 1, sp_sliding_step = 0;
    // compact schedule: resident rounds of workgroups in the grid, and 1 when
    // each XCD takes whole (kv head, head group) classes (requires
    // num_kv_heads * head_groups to be a multiple of 8)
    int compact_rounds = 8;
    int xcd_classes = 0;
};

struct Phase2Params {
    void *out;                     // [S, H, D]
    const float *exp_sums;
    const float *max_logits;
    const void *tmp_out;
    const int32_t *seq_lens;
    int num_seqs, num_heads, max_num_partitions;
};

// Host-side launchers (one per translation unit that defines the kernels).
// Return hipSuccess, or hipErrorInvalidValue for an unsupported combination.
hipError_t launch_phase1(const Phase1Params &p, int qdt, int kvdt, int head_size,
                         int waves, int lds_bytes, hipStream_t stream);
hipError_t launch_phase2(const Phase2Params &p, int odt, int head_size, int threads,
                         int lds_bytes, hipStream_t stream);
hipError_t launch_decode_kv(const void *src, float *dst, int64_t n, int dtype, int via,
                            hipStream_t stream);
hipError_t launch_read_stream(const void *src, int64_t bytes, bool nontemporal, uint32_t *sink, int workgroups,
                              hipStream_t stream);
hipError_t launch_check_inputs(const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                               int max_blocks_per_seq, int block_size, int num_blocks, long long *report,
                               hipStream_t stream);

// Phase-1 workgroup shape: wavefronts per workgroup, minimum wavefronts per
// SIMD the register budget must allow, and whether K/V loads carry the
// non-temporal (streaming) hint.
#ifndef PAV2_PHASE1_WAVES
#define PAV2_PHASE1_WAVES 4
#endif
#ifndef PAV2_PHASE1_OCCUPANCY
#define PAV2_PHASE1_OCCUPANCY 1
#endif
#ifndef PAV2_PHASE1_NONTEMPORAL
#define PAV2_PHASE1_NONTEMPORAL 1
#endif
constexpr int kPhase1Waves = PAV2_PHASE1_WAVES;
#ifndef PAV2_PREFIX_SLICE
#define PAV2_PREFIX_SLICE 512
#endif
// Prefix attention: rows (query token, head) per workgroup, 16 per
// wavefront, and the key slice every wavefront walks per step (32-token
// units; a divisor of the partition).  A whole partition per step halves
// the per-step max reduction and rescale against 256 tokens and keeps more
// loads in flight; the bf16 d = 256 kernel then holds about 400 registers
// (one wavefront per SIMD, no spills).
constexpr int kPrefixRows = kPhase1Waves * kMaxHeadsPerGroup;
constexpr int kPrefixSlice = PAV2_PREFIX_SLICE;
static_assert(kPrefixSlice % 32 == 0 && kPartition % kPrefixSlice == 0, "prefix slice: 32-token units dividing the partition");
constexpr int kPhase1Occupancy = PAV2_PHASE1_OCCUPANCY;
constexpr bool kPhase1NonTemporal = PAV2_PHASE1_NONTEMPORAL != 0;
constexpr int kPhase2Threads = 256;

// Phase-1 schedule: 0 dense grid, 1 compact list of used partitions, 2 choose
// (compact for batches of 2 .. kMaxCompactSeqs sequences).
#ifndef PAV2_PHASE1_SCHEDULE
#define PAV2_PHASE1_SCHEDULE 2
#endif
constexpr int kMaxCompactSeqs = 8192;
#ifndef PAV2_PHASE1_COMPACT_ROUNDS
#define PAV2_PHASE1_COMPACT_ROUNDS 8
#endif
constexpr int kPhase1CompactRounds = PAV2_PHASE1_COMPACT_ROUNDS;
// 1: the compact grid's workgroups on one XCD (blockIdx % 8) take one
// contiguous block of the item list, so each XCD's L2 holds the output rows
// and block-table entries of neighbouring items.
#ifndef PAV2_PHASE1_XCD_RANGES
#define PAV2_PHASE1_XCD_RANGES 1
#endif
constexpr int kPhase1XcdRanges = PAV2_PHASE1_XCD_RANGES;
// Batches of many sequences (kPhase1ManySeqs or more): every compact-schedule
// workgroup first scans all sequences' partition counts, so the grid is one
// resident round (a scan per resident slot, each workgroup then walking a
// longer balanced range), and when the (kv head, head group) classes are a
// multiple of 8 each XCD takes whole classes: XCD x walks the (sequence,
// partition) lists of classes x * C/8 .. (x + 1) * C/8 - 1, split among its
// workgroups.  Measured on the MI355X against 8 rounds in item order:
// 256 ragged sequences (d = 80, 8 kv heads) 65.2 -> 67.1 % of HBM peak, 32
// sequences of 512-4096 tokens (d = 128, 8 kv heads) 61.3 -> 62.0 %; a
// batch of 4 long sequences loses with one round (73.8 -> 70.5 %: 6.1
// uniform items per workgroup leave a 14 % tail), so it keeps 8 rounds and
// the hardware dispatcher's balance.
constexpr int kPhase1ManySeqs = 16;
inline int phase1_compact_rounds(int num_seqs) { return num_seqs >= kPhase1ManySeqs ? 1 : kPhase1CompactRounds; }
inline bool phase1_xcd_classes(int num_seqs, int num_kv_heads, int head_groups) {
    return num_seqs >= kPhase1ManySeqs && (num_kv_heads * head_groups) % 8 == 0;
}

inline bool phase1_compact(int num_seqs) {
    if (PAV2_PHASE1_SCHEDULE == 0) return false;
    if (num_seqs > kMaxCompactSeqs) return false;
    return PAV2_PHASE1_SCHEDULE == 1 || num_seqs > 1;
}

// Dispatch between the single-pass kernel and the two-phase path: single
// pass when every sequence fits one partition (no combine needed), or when the
// (sequence, kv head, head group) workgroups alone give every compute unit
// two or more and no sequence spans more than 32 partitions (a workgroup then
// streams up to 16K tokens without the per-partition outputs, the second
// launch and its gap; for equal lengths it is the faster path, e.g. 64 x 16K
// tokens with an e4m3 cache: 0.325 ms single pass against 0.399 ms for the
// two phases).  Decided from the shapes alone (no read of seq_lens), as the
// pages' own rule is; a batch that puts one long sequence among many short
// ones walks that sequence's partitions serially.  Planned for the MI355X's
// 256 compute units, without querying the device.
constexpr int kPlanCUs = 256;
constexpr int kSinglePassMinRounds = 2;      // workgroups >= this many per CU
constexpr int kSinglePassMaxPartitions = 32; // and at most this many partitions per sequence
inline bool prefer_single_pass(int64_t seq_items, int max_num_partitions) {
    if (max_num_partitions <= 1) return true;
    return seq_items >= (int64_t)kSinglePassMinRounds * kPlanCUs &&
           max_num_partitions <= kSinglePassMaxPartitions;
}

inline int phase1_lds_bytes(int gqa, int head_size, int waves, int bs_log2, int num_seqs, bool compact,
                            bool sparse = false) {
    int heads = gqa < kMaxHeadsPerGroup ? gqa : kMaxHeadsPerGroup;
    int d16 = (head_size + 15) / 16 * 16;
    int table = (kPartition >> bs_log2) * 4;
    return waves * heads * (d16 + 4) * 4      // per-wave partial outputs
           + 3 * waves * kMaxHeadsPerGroup * 4 // per-wave max and sums
           + table * (sparse ? waves : 1)      // the partition's block-table slice (block-sparse: one per wavefront)
           + (num_seqs + 1 + waves) * 4 * (compact ? 1 : 0)   // partition-count prefix
           + (sparse ? (kMaxHeadsPerGroup + waves) * 4 : 0);   // heads' stripe residues, unit masks
}

inline int phase2_vec(int odt) { return odt == F32 ? 4 : 8; }

inline int phase2_lds_bytes(int max_num_partitions, int head_size, int odt) {
    (void)max_num_partitions, (void)head_size, (void)odt;
    return 0;   // phase 2 keeps everything in registers
}

// Wavefronts phase 2 gives one (sequence, head): one for up to 64 partition
// slots (a workgroup serves four pairs), 4 up to 128, 16 beyond (one
// workgroup of that many wavefronts per pair).
inline int phase2_waves_per_pair(int max_num_partitions) {
    return max_num_partitions > 128 ? 16 : (max_num_partitions > 64 ? 4 : 1);
}

// Short contexts with more (sequence, head) pairs than one resident round of
// wavefronts (4 per SIMD on 256 compute units) give each wavefront two
// pairs, 32 lanes each, so that every pair's chain of dependent reads runs in
// one round (at the cost of one more row batch for the longest contexts).
constexpr int64_t kPhase2OneRoundWaves = 256 * 16;
inline int phase2_pairs_per_wave(int64_t pairs, int max_num_partitions, int head_size, int odt) {
    const int lanes_per_row = head_size / (odt == F32 ? 4 : 8);   // a row must fit the pair's 32 lanes
    return phase2_waves_per_pair(max_num_partitions) == 1 && pairs > kPhase2OneRoundWaves && lanes_per_row <= 32
               ? 2 : 1;
}
inline int phase2_workgroups(int64_t pairs, int max_num_partitions, int head_size, int odt) {
    const int wpp = phase2_waves_per_pair(max_num_partitions);
    const int ppw = phase2_pairs_per_wave(pairs, max_num_partitions, head_size, odt);
    const int wg_waves = wpp > 4 ? wpp : 4;
    const int64_t waves = (pairs + ppw - 1) / ppw * wpp;
    return (int)((waves + wg_waves - 1) / wg_waves);
}

}  // namespace pav2
