// Paged prefix attention (chunked prefill) on gfx950 for 16-bit caches:
// the query rows of each sequence's new chunk against its cached context
// and, causally, the chunk itself, all read from the paged cache (page
// "paged_attn.py", _forward_prefix_pytorch: context tiles without a mask,
// then the current chunk with the causal mask, merged by an online softmax;
// tiling the keys re-associates one softmax over every visible key).
//
//   out[q0 + j, h] = softmax_t(scale * q . K_t) V_t,  t < ctx + j + 1,
//
// with K_t, V_t of kv head h / gqa gathered through block_tables[s].
//
// Mapping onto CDNA4 (a dense contraction, so MFMA-bound by design):
// * One workgroup (4 wavefronts) per (sequence, kv head, block of 128 rows),
//   row rr = token j * gqa + head r of the chunk; wavefront w owns rows
//   32 w .. 32 w + 31.  All rows of a block share the kv head's keys.
// * Keys are taken 64 at a time.  Each tile of K and V is copied once per
//   workgroup from the paged cache into LDS with gfx950's 16-byte direct
//   global->LDS loads (no registers on the way), double-buffered: the copy of
//   tile t + 1 runs while tile t is multiplied.  K is stored as 16-byte
//   vectors [head-dim chunk][key] (a key's 8 consecutive head-dim elements,
//   as in the cache), V as [8-key group][head-dim row] (8 consecutive keys
//   of one row, as in the cache); both read back conflict-free.
// * S^T = K Q^T on 32x32x16 MFMA tiles (32 keys x 32 query rows, contraction
//   over the head dimension): the A operand is one 16-byte K vector per
//   lane, the B operand the lane's query row held in registers for the
//   whole run.  The accumulator gives every lane one query row, so the
//   running max and the rescale are per-lane scalars.
// * O^T = V^T P^T, also 32x32x16: A = 8 keys of one V row (one 16-byte LDS
//   vector), B = the lane's row of P.  One v_permlane32_swap per pair of
//   packed registers moves the accumulator's key order (4 keys per half-wave
//   per group of 8) into the B operand's (8 consecutive keys per half-wave).
// * Online softmax with a lazy rescale: the running offset moves only when a
//   tile's maximum exceeds it by more than 8 (log2 units), so weights stay
//   below 2^8 and most tiles skip the rescale of the 32 x D accumulators.
//   The weights enter the MFMA rounded to 16 bits (bfloat16: as a hi + lo
//   pair of 16-bit parts, two MFMAs) and their sum is taken over the values
//   as rounded, so the output is an exact weighted mean of V rows under the
//   weights the MFMAs saw.
#include <math.h>

#include "pav2_internal.h"
#include "prefix.h"

namespace pav2 {
namespace {

constexpr int kRows = 128;     // query rows per workgroup (4 wavefronts x 32)
constexpr int kKeys = 64;      // keys per tile
constexpr float kLazy = 8.0f;  // log2 headroom before the running offset moves
constexpr int kPre = 4;        // LDS fragment reads issued ahead of the MFMAs

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lds_ptr;

template <int N>
struct IC {   // a compile-time int argument for generic lambdas
    static constexpr int value = N;
};

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8v, a), __builtin_bit_cast(f16x8v, b),
                                                      c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
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

// Element E (0: low, 1: high) of a packed pair of 16-bit values, as float.
template <int DT, int E>
__device__ __forceinline__ float unpack16(uint32_t w) {
    if constexpr (DT == BF16) return as_f32(E ? (w & 0xffff0000u) : (w << 16));
    else return (float)as_f16x2(w)[E];
}

// SPLIT: the weights enter P V as two 16-bit parts (hi + the rounding
// residual, ~16 significant bits); bfloat16's 8-bit significand alone moves
// the output of rows with few visible keys by more than the tolerance.
template <int DT, int D, bool SPLIT = (DT == BF16)>
__global__ void __launch_bounds__(256) prefix_kernel(const PrefixParams P) {
    static_assert(D % 32 == 0 && D <= 256, "head size: whole 32-row output tiles");
    constexpr int NC = D / 8;                 // 16-byte K chunks per token
    constexpr int NS = D / 16;                // QK contraction steps
    constexpr int NDT = D / 32;               // O^T tiles (32 head-dim rows each)
    constexpr int TILE = D * kKeys * 2;       // bytes of one K (or V) tile
    constexpr int VI = (D + 63) / 64;         // V copies (64 rows each) per 8-key group
    constexpr int KPW = NC / 4;               // K copies per wavefront per tile
    constexpr int VPW = 2 * VI;               // V copies per wavefront per tile
    static_assert(NC % 4 == 0, "K copies split over 4 wavefronts");
    __shared__ __align__(16) uint8_t k0[TILE], k1[TILE], v0[TILE], v1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, lrow = lane & 31;

    // workgroups numbered XCD by XCD (grid a multiple of 8; blockIdx % 8 picks
    // the XCD), so the row blocks of one (sequence, kv head) share an L2
    const int wg = (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3));
    if (wg >= P.num_work) return;
    const int RB = P.row_blocks, KVH = P.num_kv_heads, gqa = P.gqa;
    const int s = wg / (KVH * RB), g = (wg / RB) % KVH, rb = wg % RB;
    const int q0 = P.query_start_loc[s];
    const int nrows = (P.query_start_loc[s + 1] - q0) * gqa;
    const int ctx = P.context_lens[s];
    if (rb * kRows >= nrows) return;
    const int Lmax = ctx + (min(nrows, (rb + 1) * kRows) - 1) / gqa + 1;   // the block's largest limit
    const int lmin = ctx + (rb * kRows) / gqa + 1;                          // its smallest
    const int ntiles = (Lmax + kKeys - 1) / kKeys;

    // this lane's query row and its causal limit (keys t < lim)
    const int row = rb * kRows + wv * 32 + lrow;
    const bool rvalid = row < nrows;
    const int jq = row / gqa, rq = row - jq * gqa;
    const int lim = rvalid ? ctx + jq + 1 : Lmax;

    // zero the tiles once: keys past the block's limit are never copied, and
    // what their slots hold must be finite (they meet zero weights)
    for (int i = tid; i < TILE / 16; i += 256) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        reinterpret_cast<u32x4 *>(k0)[i] = z;
        reinterpret_cast<u32x4 *>(k1)[i] = z;
        reinterpret_cast<u32x4 *>(v0)[i] = z;
        reinterpret_cast<u32x4 *>(v1)[i] = z;
    }

    // query fragments (B operand of S^T = K Q^T): row lrow, head-dim 16 s + 8 half .. + 7
    u32x4 qf[NS];
    {
        const uint8_t *qrow = reinterpret_cast<const uint8_t *>(P.query) +
                              ((int64_t)(q0 + jq) * P.num_heads + g * gqa + rq) * D * 2;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (rvalid) v = *reinterpret_cast<const u32x4 *>(qrow + (16 * st + 8 * half) * 2);
            qf[st] = v;
        }
    }

    const int bs_log2 = P.bs_log2;
    const int bs_mask = (1 << bs_log2) - 1;
    const int32_t *bt = P.block_tables + (int64_t)s * P.max_blocks_per_seq;
    const uint8_t *kc = P.key_cache + (int64_t)g * P.head_stride;
    const uint8_t *vc = P.value_cache + (int64_t)g * P.head_stride;
    const int64_t blk_stride = P.blk_stride;

    // block of key t0 + lane of a tile (lanes past the limit: 0, never used)
    auto key_block = [&](int t) -> int {
        const int key = t * kKeys + lane;
        return key < Lmax ? bt[key >> bs_log2] : 0;
    };
    // copy tile t into (kd, vd): this wavefront's K chunks and V rows
    auto copy_tile = [&](int t, int blk, uint8_t *kd, uint8_t *vd) {
        const int t0 = t * kKeys;
        const int key = t0 + lane;
#pragma unroll
        for (int k = 0; k < KPW; ++k) {
            const int c = wv * KPW + k;
            if (key < Lmax) {
                const uint8_t *src = kc + (int64_t)blk * blk_stride + (((int64_t)c << bs_log2) + (key & bs_mask)) * 16;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(kd + c * kKeys * 16), 16, 0, 0);
            }
        }
#pragma unroll
        for (int k = 0; k < VPW; ++k) {
            const int ki = wv * VPW + k;
            const int kg = ki / VI, d0 = (ki % VI) * 64;
            const int d = d0 + lane;
            // the group's 8 keys share one block (block sizes >= 8 here)
            const int gb = __builtin_amdgcn_readlane(blk, 8 * kg);
            if (8 * kg < Lmax - t0 && d < D) {
                const uint8_t *src = vc + (int64_t)gb * blk_stride +
                                     (((int64_t)d << bs_log2) + ((t0 + 8 * kg) & bs_mask)) * 2;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)(vd + (kg * D + d0) * 16), 16, 0, 0);
            }
        }
    };

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
    float lsum = 0.0f;          // this half-wave's share of the row's rounded-weight sum
    float m_used = -INFINITY;   // running offset (log2 units) of the weights
    const float sl2 = P.scale_log2;

    // one tile, as two halves of 32 keys: S^T, mask, max, weights, O^T
    auto compute = [&](int t, const uint8_t *kb, const uint8_t *vb) {
        const int t0 = t * kKeys;
        const uint8_t *kl = kb + (half * kKeys + lrow) * 16;   // A of S^T: key 32 nt + lrow, chunk 2 st + half
        const uint8_t *vl = vb + (half * D + lrow) * 16;       // A of O^T: group 2 ks + half, row 32 dt + lrow
        auto half_tile = [&](auto ntc) {
            constexpr int nt = decltype(ntc)::value;
            f32x16 acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(kl + (2 * st * kKeys + 32 * nt) * 16);
                acc = mfma32<DT>(a, qf[st], acc);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, kPre, 2 * nt);   // kPre LDS reads ahead
#pragma unroll
            for (int f = 0; f < NS - kPre; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 2 * nt);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 2 * nt);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kPre, 2 * nt);

            // element i: key t0 + 32 nt + 8 (i / 4) + 4 half + i % 4; the
            // scale (> 0) is applied with the offset, in one FMA per weight
            if (t0 + 32 * nt + 32 > lmin) {   // the half reaches some row's causal limit (uniform)
                const int rel = lim - t0 - 32 * nt - 4 * half;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = (8 * (i / 4) + (i % 4)) < rel ? acc[i] : -INFINITY;
            }
            float mx = acc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;   // the other half-wave holds the row's other keys
            if (mx > m_used + kLazy) {   // move the offset; rescale what was accumulated
                const float alpha = __builtin_amdgcn_exp2f(m_used - mx);   // 0 on the first visible keys
                m_used = mx;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
                lsum *= alpha;
            }
            const float mu = m_used == -INFINITY ? 0.0f : m_used;
            const float nmu = -mu;

#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {   // the half's two steps of 16 keys (k-groups ke, ko)
                const int ks = 2 * nt + kh, ke = 2 * kh, ko = ke + 1;
                float pv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = __builtin_amdgcn_exp2f(fmaf(acc[4 * ke + i], sl2, nmu));
                    pv[4 + i] = __builtin_amdgcn_exp2f(fmaf(acc[4 * ko + i], sl2, nmu));
                }
                uint32_t w[4] = {pack16<DT>(pv[0], pv[1]), pack16<DT>(pv[2], pv[3]), pack16<DT>(pv[4], pv[5]),
                                 pack16<DT>(pv[6], pv[7])};
                uint32_t r[4] = {0u, 0u, 0u, 0u};
                if constexpr (SPLIT) {   // the rounding residual as a second 16-bit part
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        r[k] = pack16<DT>(pv[2 * k] - unpack16<DT, 0>(w[k]), pv[2 * k + 1] - unpack16<DT, 1>(w[k]));
                }
                // sum of the weights as they enter the MFMAs: one 16-bit part
                // each -- or hi + lo, equal to the float32 weight to ~2^-17
                if constexpr (SPLIT) {
                    lsum += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) lsum += unpack16<DT, 0>(w[k]) + unpack16<DT, 1>(w[k]);
                }
                // half 0 held keys 0-3 and 8-11 of the step, half 1 keys 4-7 and
                // 12-15: one swap per register pair gives half h keys 8 h .. 8 h + 7
                auto regroup = [](uint32_t (&x)[4]) {
                    const auto a0 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
                    const auto a1 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
                    x[0] = a0[0];
                    x[2] = a0[1];
                    x[1] = a1[0];
                    x[3] = a1[1];
                };
                regroup(w);
                if constexpr (SPLIT) regroup(r);
                const u32x4 pb = {w[0], w[1], w[2], w[3]};
                const u32x4 pl = {r[0], r[1], r[2], r[3]};
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(vl + (2 * ks * D + 32 * dt) * 16);
                    o[dt] = mfma32<DT>(a, pb, o[dt]);
                    if constexpr (SPLIT) o[dt] = mfma32<DT>(a, pl, o[dt]);
                }
            }
            constexpr int MPF = SPLIT ? 2 : 1;   // MFMAs per V fragment
            constexpr int VPRE = kPre < 2 * NDT ? kPre : 2 * NDT;
            __builtin_amdgcn_sched_group_barrier(0x100, VPRE, 2 * nt + 1);
#pragma unroll
            for (int f = 0; f < 2 * NDT - VPRE; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, MPF, 2 * nt + 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 2 * nt + 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MPF * VPRE, 2 * nt + 1);
        };
        half_tile(IC<0>{});
        half_tile(IC<1>{});
    };

    // the last tile's partial 8-key group: V of keys past the block's limit
    // (other sequences' data or unwritten slots) is zeroed in LDS before use,
    // as it meets zero weights and must not be NaN
    auto zero_tail = [&](int t, uint8_t *vb) {
        const int nv = Lmax - t * kKeys;   // valid keys of the tile
        if (nv >= kKeys || (nv & 7) == 0) return;
        const int kg = nv >> 3, keep = nv & 7;
        for (int d = tid; d < D; d += 256) {
            u32x4 *vp = reinterpret_cast<u32x4 *>(vb + (kg * D + d) * 16);
            u32x4 v = *vp;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t m = (2 * q + 1 < keep) ? ~0u : (2 * q < keep ? 0xffffu : 0u);
                v[q] &= m;
            }
            *vp = v;
        }
    };

    // pipeline: copy t + 1 while computing t; the barrier at the top of each
    // step finds every wavefront's copies of that tile landed and the other
    // buffer free
    int blk = key_block(0);
    __syncthreads();   // the zeroed tiles are in place before any copy lands
    copy_tile(0, blk, k0, v0);
    blk = ntiles > 1 ? key_block(1) : 0;
    for (int t = 0; t < ntiles; t += 2) {
        __syncthreads();
        if (t + 1 == ntiles) {   // last tile (uniform)
            zero_tail(t, v0);
            __syncthreads();
        }
        if (t + 1 < ntiles) copy_tile(t + 1, blk, k1, v1);
        blk = t + 2 < ntiles ? key_block(t + 2) : 0;
        compute(t, k0, v0);
        if (t + 1 >= ntiles) break;
        __syncthreads();
        if (t + 2 == ntiles) {
            zero_tail(t + 1, v1);
            __syncthreads();
        }
        if (t + 2 < ntiles) copy_tile(t + 2, blk, k0, v0);
        blk = t + 3 < ntiles ? key_block(t + 3) : 0;
        compute(t + 1, k1, v1);
    }

    // normalise and store: lane holds row lrow, head-dim 32 dt + 8 (i / 4) + 4 half + i % 4
    if (!rvalid) return;
    const float lr = lsum + __shfl_xor(lsum, 32);   // both half-waves' keys
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    uint8_t *orow = reinterpret_cast<uint8_t *>(P.out) + ((int64_t)(q0 + jq) * P.num_heads + g * gqa + rq) * D * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int d = 32 * dt + 8 * q + 4 * half;
            const u32x2 w = {pack16<DT>(o[dt][4 * q + 0] * inv, o[dt][4 * q + 1] * inv),
                             pack16<DT>(o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv)};
            *reinterpret_cast<u32x2 *>(orow + d * 2) = w;
        }
}

template <int DT>
hipError_t launch_dt(const PrefixParams &p, int head_size, hipStream_t stream) {
    const dim3 grid((unsigned)((p.num_work + 7) / 8 * 8)), block(256);
    switch (head_size) {
    case 64: hipLaunchKernelGGL((prefix_kernel<DT, 64>), grid, block, 0, stream, p); break;
    case 96: hipLaunchKernelGGL((prefix_kernel<DT, 96>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((prefix_kernel<DT, 128>), grid, block, 0, stream, p); break;
    case 192: hipLaunchKernelGGL((prefix_kernel<DT, 192>), grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL((prefix_kernel<DT, 256>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool prefix_mfma_supported(int dtype, int head_size, int bs_log2, float scale) {
    return (dtype == F16 || dtype == BF16) && head_size % 32 == 0 && head_size <= 256 && bs_log2 >= 3 &&
           scale > 0.0f;
}

hipError_t launch_prefix(const PrefixParams &p, int dtype, int head_size, hipStream_t stream) {
    if (!prefix_mfma_supported(dtype, head_size, p.bs_log2, p.scale_log2)) return hipErrorInvalidValue;
    return dtype == BF16 ? launch_dt<BF16>(p, head_size, stream) : launch_dt<F16>(p, head_size, stream);
}

}  // namespace pav2
