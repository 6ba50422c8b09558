// KV-cache write: launch parameters shared by the C ABI and the kernel.
#pragma once

#include "pav2_internal.h"

namespace pav2 {

struct CacheParams {
    const uint8_t *key;            // [T, KVH, D] input dtype
    const uint8_t *value;          // [T, KVH, D]
    uint8_t *key_cache;            // [NB, KVH, D/x, BS, x] cache dtype
    uint8_t *value_cache;          // [NB, KVH, D, BS]
    const int64_t *slot_mapping;   // [T]
    int num_tokens, num_kv_heads, head_size;
    int bs_log2;                   // log2(block_size)
    int64_t num_slots;             // num_blocks * block_size
    int64_t blk_stride;            // bytes per physical block (all kv heads)
    int64_t head_stride;           // bytes per (block, kv head)
    float k_scale, v_scale;        // the write divides by these
    float k_rcp, v_rcp;            // RN(1 / scale), for the FMA-corrected quotient
    int fast_div;                  // 1: both reciprocals are normal floats (scales in [2^-100, 2^100])
};

// Returns hipSuccess, or hipErrorInvalidValue for an unsupported combination.
hipError_t launch_cache_write(const CacheParams &p, int input_dtype, int cache_dtype, hipStream_t stream);

}  // namespace pav2
