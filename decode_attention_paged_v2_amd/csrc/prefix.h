// Paged prefix attention on MFMA tiles: launch parameters shared by the C ABI
// and the kernel (csrc/prefix.hip).
#pragma once

#include "pav2_internal.h"

namespace pav2 {

struct PrefixParams {
    void *out;                       // [T, H, D] dtype
    const void *query;               // [T, H, D]
    const uint8_t *key_cache;        // [NB, KVH, D/8, BS, 8]
    const uint8_t *value_cache;      // [NB, KVH, D, BS]
    const int32_t *block_tables;     // [S, MBPS]
    const int32_t *query_start_loc;  // [S + 1]
    const int32_t *context_lens;     // [S]
    int num_seqs, num_heads, num_kv_heads, gqa;
    int row_blocks;                  // ceil(max_query_len * gqa / 128)
    int bs_log2, max_blocks_per_seq;
    int num_work;                    // num_seqs * num_kv_heads * row_blocks
    int64_t blk_stride, head_stride;
    float scale_log2;                // scale * log2(e)
    // every byte of a kv head's cache slab lies within 4 GiB of the slab's
    // first block (num_blocks * blk_stride <= 2^32): the tiles are then copied
    // with buffer (32-bit offset) loads into LDS, else with global ones
    bool offsets32;
    // key ranges per row block: 1 writes the output directly; more split each
    // row block's tiles into that many ranges whose normalised partial
    // outputs (float32) and statistics go to `part`, merged by a second kernel
    int splits = 1;
    // o: per (range, row block) item [D / 4][128 rows][4] floats, then m and
    // l: [splits * num_work * 128] floats each
    float *part = nullptr;
};

constexpr int kPrefixMfmaRows = 128;   // query rows per workgroup

// Whether the MFMA-tile kernel serves this case (16-bit caches, head size a
// multiple of 32, blocks of at least 8 tokens, a positive scale); others take
// phase 1's prefix schedule.
bool prefix_mfma_supported(int dtype, int head_size, int bs_log2, float scale);
// Key ranges per row block (1 .. kPrefixMaxSplits) that balance this launch
// over the current device's compute units, from the kernel's occupancy; 1
// when splitting does not shorten the estimated run.
constexpr int kPrefixMaxSplits = 8;
int prefix_splits(int dtype, int head_size, bool offsets32, int num_work, int max_seq_len);
// Workspace bytes for `splits` ranges (0 for one).
size_t prefix_workspace_bytes(int splits, int num_work, int head_size);
hipError_t launch_prefix(const PrefixParams &p, int dtype, int head_size, hipStream_t stream);

}  // namespace pav2
