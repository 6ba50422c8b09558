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

#include <map>
#include <mutex>
#include <utility>

#include "pav2_internal.h"
#include "prefix.h"

namespace pav2 {
namespace {

constexpr int kRows = 128;     // query rows per workgroup (4 wavefronts x 32)
constexpr int kKeys = 64;      // keys per tile
constexpr float kLazy = 8.0f;  // log2 headroom before the running offset moves

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lds_ptr;

template <int N>
struct IC {   // a compile-time int argument for generic lambdas
    static constexpr int value = N;
};

// f(IC<I>{}), f(IC<I + 1>{}), ..., f(IC<N - 1>{})
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(IC<I>{});
        static_for<I + 1, N>(f);
    }
}

// Wait until every copy this wavefront issued into LDS has landed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left alone).  A barrier publishes
// LDS writes, but the compiler treats a copy into LDS as a load whose result
// only its own wavefront needs and may leave it in flight across the barrier,
// so every barrier that hands copied tiles to the other wavefronts follows
// this wait.
__device__ __forceinline__ void copies_landed() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
// BUF: the tiles are copied with buffer loads (32-bit offsets from the kv
// head's slab, which must span at most 4 GiB).  The compiler counts a global
// load into LDS as a possible LDS access of its own and so waits for every
// outstanding LDS read wherever one is pending; with buffer loads its waits
// for the fragment reads stay partial (the hardware counts neither form
// against the LDS counter).
template <int DT, int D, bool BUF, bool SPLIT = (DT == BF16)>
__global__ void __launch_bounds__(256) prefix_kernel(const PrefixParams P) {
    static_assert(D % 32 == 0 && D <= 256, "head size: whole 32-row output tiles");
    constexpr int NC = D / 8;                 // 16-byte K chunks per token
    constexpr int NS = D / 16;                // QK contraction steps
    constexpr int NDT = D / 32;               // O^T tiles (32 head-dim rows each)
    constexpr int TILE = D * kKeys * 2;       // bytes of one K (or V) tile
    constexpr int VI = (D + 63) / 64;         // V copies (64 rows each) per 8-key group
    constexpr int KPW = NC / 4;               // K copies per wavefront per tile
    constexpr int VPW = 2 * VI;               // V copies per wavefront per tile
    constexpr int SW = NS % 2 == 0 ? 2 : 1;   // contraction steps per pipeline slot
    constexpr int NSLOT = NS / SW;            // slots per 32-key step
    static_assert(NC % 4 == 0, "K copies split over 4 wavefronts");
    __shared__ __align__(16) uint8_t k0[TILE], k1[TILE], v0[TILE], v1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, lrow = lane & 31;

    // workgroups numbered XCD by XCD (grid a multiple of 8; blockIdx % 8 picks
    // the XCD), so the row blocks of one (sequence, kv head) share an L2
    const int item = (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3));
    if (item >= P.num_work * P.splits) return;
    const int split = item / P.num_work, wg = item - split * P.num_work;   // key range, row block
    const int RB = P.row_blocks, KVH = P.num_kv_heads, gqa = P.gqa;
    const int s = wg / (KVH * RB), g = (wg / RB) % KVH, rb = wg % RB;
    const int q0 = P.query_start_loc[s];
    const int nrows = (P.query_start_loc[s + 1] - q0) * gqa;
    const int ctx = P.context_lens[s];
    if (rb * kRows >= nrows) return;
    const int Lmax = ctx + (min(nrows, (rb + 1) * kRows) - 1) / gqa + 1;   // the block's largest limit
    const int lmin = ctx + (rb * kRows) / gqa + 1;                          // its smallest
    const int ntiles = (Lmax + kKeys - 1) / kKeys;
    // this item's tiles [tb, te): range `split` of the row block's
    const int tper = (ntiles + P.splits - 1) / P.splits;
    const int tb = split * tper, te = min(ntiles, tb + tper);

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
    // buffer resources over the kv head's slabs (raw, byte offsets, 32-bit
    // data format word as gfx9 wants; no range limit below 4 GiB)
    __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(kc), 0, -1, 0x00020000);
    __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(vc), 0, -1, 0x00020000);

    // block of key t * kKeys + lane, clamped to the block's last key: every
    // K slot of a copied tile holds a real (finite) key; the surplus ones meet
    // the causal mask
    auto key_block = [&](int t) -> int { return bt[min(t * kKeys + lane, Lmax - 1) >> bs_log2]; };
    // one copy instruction of a tile: K chunk row wv * KPW + k (64 keys x 16
    // bytes), or V instruction k of this wavefront (64 head-dim rows of one
    // 8-key group)
    auto copy_k_one = [&](int k, int t, int blk, uint8_t *kd) __attribute__((always_inline)) {
        const int key = min(t * kKeys + lane, Lmax - 1);
        const int c = wv * KPW + k;
        const int64_t off = (int64_t)blk * blk_stride + (((int64_t)c << bs_log2) + (key & bs_mask)) * 16;
        if constexpr (BUF)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr)(kd + c * kKeys * 16), 16, (uint32_t)off, 0, 0, 0);
        else
            __builtin_amdgcn_global_load_lds(kc + off, (lds_ptr)(kd + c * kKeys * 16), 16, 0, 0);
    };
    // V: groups of 8 keys (one block each, as block sizes are >= 8); a group
    // past the block's limit takes the last group that holds a key below it,
    // and the last tile's keys past the limit are zeroed before use
    auto copy_v_one = [&](int k, int t, int blk, uint8_t *vd) __attribute__((always_inline)) {
        const int t0 = t * kKeys;
        const int ki = wv * VPW + k;
        const int kg = ki / VI, d0 = (ki % VI) * 64;
        const int d = d0 + lane;
        const int kgs = min(kg, (Lmax - 1 - t0) >> 3);   // source group (uniform)
        const int gb = __builtin_amdgcn_readlane(blk, 8 * kgs);
        if (D % 64 == 0 || d < D) {   // (head sizes of 64 k + 32: the last copy's upper half-wave idles)
            const int64_t off = (int64_t)gb * blk_stride + (((int64_t)d << bs_log2) + ((t0 + 8 * kgs) & bs_mask)) * 2;
            if constexpr (BUF)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr)(vd + (kg * D + d0) * 16), 16, (uint32_t)off, 0, 0,
                                                         0);
            else
                __builtin_amdgcn_global_load_lds(vc + off, (lds_ptr)(vd + (kg * D + d0) * 16), 16, 0, 0);
        }
    };
    auto copy_k = [&](int t, int blk, uint8_t *kd) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < KPW; ++k) copy_k_one(k, t, blk, kd);
    };
    auto copy_v = [&](int t, int blk, uint8_t *vd) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < VPW; ++k) copy_v_one(k, t, blk, vd);
    };

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
    float lsum = 0.0f;          // this half-wave's share of the row's weight sum
    float m_used = -INFINITY;   // running offset (log2 units) of the weights
    const float sl2 = P.scale_log2;
    f32x16 s_cur;               // raw scores S^T of the half being turned into weights
    u32x4 p_prev[2][2];         // [16-key step][hi, lo]: weights of the half whose P.V is pending
    const int koff = (half * kKeys + lrow) * 16;   // A of S^T: key 32 nt + lrow, chunk 2 st + half
    const int voff = (half * D + lrow) * 16;       // A of O^T: group 2 ks + half, row 32 dt + lrow
    // this lane's fragment base in each buffer, held in a register the
    // compiler does not fold back into constants, so every fragment read adds
    // its offset (< 64 KiB) in the instruction (the buffers span 4 x D x 128
    // bytes); the pointer stays derived from its buffer for alias analysis
    auto lane_base = [&](uint8_t *buf, int off) -> const uint8_t * {
        const uint32_t a = (uint32_t)(uintptr_t)(lds_ptr)buf;
        uint32_t x = a + (uint32_t)off;
        asm volatile("" : "+v"(x));
        return buf + (x - a);
    };
    const uint8_t *const kl0 = lane_base(k0, koff), *const kl1 = lane_base(k1, koff);
    const uint8_t *const vl0 = lane_base(v0, voff), *const vl1 = lane_base(v1, voff);

    // the weights of one half from its scores, offset by -nmu (log2 units):
    // element i of s is key 8 (i / 4) + 4 half + i % 4 of the half; returns
    // this half-wave's sum of the weights as they enter the MFMAs
    auto weights = [&](const f32x16 &s, float nmu, u32x4 (&p)[2][2]) __attribute__((always_inline)) -> float {
        float part = 0.0f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {   // the half's two steps of 16 keys (k-groups ke, ko)
            const int ke = 2 * kh, ko = ke + 1;
            float pv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = __builtin_amdgcn_exp2f(fmaf(s[4 * ke + i], sl2, nmu));
                pv[4 + i] = __builtin_amdgcn_exp2f(fmaf(s[4 * ko + i], sl2, nmu));
            }
            uint32_t w[4] = {pack16<DT>(pv[0], pv[1]), pack16<DT>(pv[2], pv[3]), pack16<DT>(pv[4], pv[5]),
                             pack16<DT>(pv[6], pv[7])};
            uint32_t r[4] = {0u, 0u, 0u, 0u};
            if constexpr (SPLIT) {   // the rounding residual as a second 16-bit part
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    r[k] = pack16<DT>(pv[2 * k] - unpack16<DT, 0>(w[k]), pv[2 * k + 1] - unpack16<DT, 1>(w[k]));
                // hi + lo equals the float32 weight to ~2^-17: sum the weights
                part += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
            } else {   // one 16-bit part: sum the weights as rounded
#pragma unroll
                for (int k = 0; k < 4; ++k) part += unpack16<DT, 0>(w[k]) + unpack16<DT, 1>(w[k]);
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
            p[kh][0] = u32x4{w[0], w[1], w[2], w[3]};
            p[kh][1] = u32x4{r[0], r[1], r[2], r[3]};
        }
        return part;
    };

    // One step of the pipeline over 32-key halves, flags F: 1 = P.V of the
    // pending half (weights p_prev, V fragments at vl, half vnt of its tile);
    // 2 = S^T of the next half (K fragments at kl, half knt); 4 = weights of
    // half h from s_cur.  The step runs in NS slots; slot i issues the LDS
    // reads of slot i + kAhead, the MFMAs of slot i (S^T contraction step i,
    // V fragment i) and a share of the weights' VALU work, fenced so that the
    // reads keep their distance and the VALU work fills the MFMAs' shadow.
    // The rare rescale of the accumulators follows the slots.
    auto step = [&](auto flags, const uint8_t *vl, int vnt, const uint8_t *kl, int knt, int h, auto &&dma)
                    __attribute__((always_inline)) {
        constexpr int F = decltype(flags)::value;
        constexpr bool DO_PV = F & 1, DO_QK = F & 2, DO_SM = F & 4;
        if constexpr (DO_SM) {
            if (32 * h + 32 > lmin) {   // the half reaches some row's causal limit (uniform)
                const int rel = lim - 32 * h - 4 * half;
#pragma unroll
                for (int i = 0; i < 16; ++i) s_cur[i] = (8 * (i / 4) + (i % 4)) < rel ? s_cur[i] : -INFINITY;
            }
        }
        auto kfrag = [&](int i) { return *reinterpret_cast<const u32x4 *>(kl + (2 * i * kKeys + 32 * knt) * 16); };
        auto vfrag = [&](int i) {
            return *reinterpret_cast<const u32x4 *>(vl + (2 * (2 * vnt + i / NDT) * D + 32 * (i % NDT)) * 16);
        };
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
        // fragments of slot j + 1 are read while slot j multiplies: slots of
        // SW contraction steps (and SW V fragments), so each wait for LDS has
        // a slot of MFMAs and VALU work behind it
        u32x4 kr[2][SW], vr[2][SW];   // [slot parity][step in slot]
        static_for<0, SW>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (DO_QK) kr[0][j] = kfrag(j);
            if constexpr (DO_PV) vr[0][j] = vfrag(j);
        });
        // weights of the current half under the current offset: pieces 0-7
        // each turn 2 scores into a packed pair (and its residual), piece 8
        // takes the row maximum, piece 9 regroups the pairs into B operands
        const float nmu = m_used == -INFINITY ? 0.0f : -m_used;
        uint32_t w[2][4], r[2][4];
        float part = 0.0f, mxs = -INFINITY;
        u32x4 p_cur[2][2];
        auto piece = [&](auto pc) {
            constexpr int pi = decltype(pc)::value;
            if constexpr (pi < 8) {
                constexpr int kh = pi / 4, k = pi % 4;
                constexpr int i0 = k < 2 ? 4 * (2 * kh) + 2 * k : 4 * (2 * kh + 1) + 2 * (k - 2);
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s_cur[i0], sl2, nmu));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s_cur[i0 + 1], sl2, nmu));
                w[kh][k] = pack16<DT>(e0, e1);
                if constexpr (SPLIT) {   // the rounding residual as a second 16-bit part
                    r[kh][k] = pack16<DT>(e0 - unpack16<DT, 0>(w[kh][k]), e1 - unpack16<DT, 1>(w[kh][k]));
                    part += e0 + e1;   // hi + lo equals the float32 weight to ~2^-17
                } else {
                    r[kh][k] = 0u;
                    part += unpack16<DT, 0>(w[kh][k]) + unpack16<DT, 1>(w[kh][k]);   // as rounded
                }
            } else if constexpr (pi == 8) {
                float mx = s_cur[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s_cur[i]);
                const auto sw =
                    __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mxs = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;   // both half-waves' keys
            } else {
                // half 0 held keys 0-3 and 8-11 of a 16-key step, half 1 keys
                // 4-7 and 12-15: one swap per register pair gives half h keys
                // 8 h .. 8 h + 7
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const auto a0 = __builtin_amdgcn_permlane32_swap(w[kh][0], w[kh][2], false, false);
                    const auto a1 = __builtin_amdgcn_permlane32_swap(w[kh][1], w[kh][3], false, false);
                    p_cur[kh][0] = u32x4{a0[0], a1[0], a0[1], a1[1]};
                    if constexpr (SPLIT) {
                        const auto b0 = __builtin_amdgcn_permlane32_swap(r[kh][0], r[kh][2], false, false);
                        const auto b1 = __builtin_amdgcn_permlane32_swap(r[kh][1], r[kh][3], false, false);
                        p_cur[kh][1] = u32x4{b0[0], b1[0], b0[1], b1[1]};
                    } else {
                        p_cur[kh][1] = u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
        };
        static_for<0, NSLOT>([&](auto jc) {
            constexpr int j = decltype(jc)::value, cur = j & 1;
            if constexpr (j + 1 < NSLOT) {
                static_for<0, SW>([&](auto ec) {
                    constexpr int e = decltype(ec)::value;
                    if constexpr (DO_QK) kr[cur ^ 1][e] = kfrag(SW * (j + 1) + e);
                    if constexpr (DO_PV) vr[cur ^ 1][e] = vfrag(SW * (j + 1) + e);
                });
            }
            static_for<0, SW>([&](auto ec) {
                constexpr int e = decltype(ec)::value, i = SW * j + e;
                if constexpr (DO_QK) acc = mfma32<DT>(kr[cur][e], qf[i], acc);
                if constexpr (DO_PV) {
                    constexpr int kh = i / NDT, dt = i % NDT;
                    o[dt] = mfma32<DT>(vr[cur][e], p_prev[kh][0], o[dt]);
                    if constexpr (SPLIT) o[dt] = mfma32<DT>(vr[cur][e], p_prev[kh][1], o[dt]);
                }
            });
            if constexpr (DO_SM) {
                static_for<0, 10>([&](auto pc) {
                    if constexpr (decltype(pc)::value * NSLOT / 10 == j) piece(pc);
                });
            }
            dma(jc);   // this slot's share of the next tiles' copies
            // order inside the slot: the next slot's reads, then MFMAs with
            // VALU work between them (copies go where they fall)
            constexpr int NRD = j + 1 < NSLOT ? SW * ((DO_QK ? 1 : 0) + (DO_PV ? 1 : 0)) : 0;
            constexpr int NMF = SW * ((DO_QK ? 1 : 0) + (DO_PV ? (SPLIT ? 2 : 1) : 0));
            if constexpr (NRD > 0) __builtin_amdgcn_sched_group_barrier(0x100, NRD, j);
            static_for<0, NMF>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, j);
                if constexpr (DO_SM) __builtin_amdgcn_sched_group_barrier(0x002, 4, j);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (DO_SM) {
            // some row's offset moves (rare; a wave-uniform jump, so the common
            // case runs none of it): those rows rescale what they accumulated
            // and redo their weights, the others keep theirs (alpha = 1)
            const bool move = mxs > m_used + kLazy;
            if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
                const float m_new = move ? mxs : m_used;
                const float alpha = move ? __builtin_amdgcn_exp2f(m_used - mxs) : 1.0f;   // 0 on the first keys
                m_used = m_new;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
                lsum *= alpha;
                part = weights(s_cur, m_new == -INFINITY ? 0.0f : -m_new, p_cur);
            }
            lsum += part;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                p_prev[kh][0] = p_cur[kh][0];
                p_prev[kh][1] = p_cur[kh][1];
            }
        }
        if constexpr (DO_QK) s_cur = acc;
    };

    // the last tile's V past the block's limit (other sequences' data,
    // unwritten slots or copies of a group that holds them) is zeroed in LDS
    // before use, as it meets zero weights and must not be NaN
    auto zero_tail = [&](int t, uint8_t *vb) __attribute__((always_inline)) {
        const int nv = Lmax - t * kKeys;   // valid keys of the tile (1 .. 64)
        if (nv >= kKeys) return;
        const int g0 = nv >> 3;            // first group holding a key past the limit
        for (int i = tid; i < (8 - g0) * D; i += 256) {
            const int kg = g0 + i / D, d = i % D;
            const int keep = nv - 8 * kg;  // keys of the group below the limit (<= 7, maybe <= 0)
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

    // Pipeline over tiles.  Iteration T multiplies P.V of tile T's halves and
    // S^T of tile T + 1's, so it reads V(T) and K(T + 1) while the copies of
    // V(T + 1) and K(T + 2) land in the other buffers; the barrier that opens
    // it finds its tiles landed and those buffers free.  K runs one tile
    // ahead of V.  Iterations come in pairs (static buffer choice, no exit
    // between them), then the last tile's P.V.
    int blk_v = key_block(tb);  // block ids of the tile whose V is copied next
    int blk_k = 0;              // block ids of the tile whose K is copied next
    auto no_dma = [](auto) {};
    if (tb < te) {
        __syncthreads();   // the zeroed tiles are in place before any copy lands
        copy_k(tb, blk_v, k0);
        copies_landed();
        __syncthreads();
        copy_v(tb, blk_v, v0);
        blk_v = key_block(tb + 1);
        copy_k(tb + 1, blk_v, k1);   // (past the range: a buffer nothing reads)
        blk_k = key_block(tb + 2);
        step(IC<2>{}, vl0, 0, kl0, 0, 2 * tb, no_dma);       // S of the range's first half
        step(IC<6>{}, vl0, 0, kl0, 1, 2 * tb, no_dma);       // S of its second; weights of the first
    }

    auto iter = [&](auto par, int T) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        uint8_t *vnxt = PAR ? v0 : v1, *knxt = PAR ? k1 : k0;   // V(T + 1), K(T + 2)
        const uint8_t *vcur = PAR ? vl1 : vl0, *kcur = PAR ? kl0 : kl1;   // V(T), K(T + 1)
        // the copies of V(T + 1) and K(T + 2), spread over the first step's
        // slots (a burst of them would hold the wavefront's in-order issue
        // behind the texture unit's queue); the second step covers their flight
        constexpr int NCP = KPW + VPW, CPS = (NCP + NSLOT - 1) / NSLOT;
        // (K(T + 2) past the last tile copies the last key again, into a
        // buffer nothing reads: no branch in the slots)
        auto dma = [&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            static_for<j * CPS, ((j + 1) * CPS < NCP ? (j + 1) * CPS : NCP)>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                if constexpr (q < KPW) copy_k_one(q, T + 2, blk_k, knxt);
                else copy_v_one(q - KPW, T + 1, blk_v, vnxt);
            });
        };
        copies_landed();
        __syncthreads();
        step(IC<7>{}, vcur, 0, kcur, 0, 2 * T + 1, dma);
        blk_v = blk_k;
        blk_k = key_block(T + 3);
        step(IC<7>{}, vcur, 1, kcur, 1, 2 * T + 2, no_dma);
    };
    auto last = [&](auto par) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        const uint8_t *vcur = PAR ? vl1 : vl0;
        copies_landed();
        __syncthreads();
        zero_tail(te - 1, PAR ? v1 : v0);
        __syncthreads();
        step(IC<5>{}, vcur, 0, vcur, 0, 2 * te - 1, no_dma);   // P.V of half 2te-2; weights of half 2te-1
        step(IC<1>{}, vcur, 1, vcur, 0, 2 * te, no_dma);       // P.V of half 2te-1
    };
    if (tb < te) {
        int T = tb;
        for (; T + 2 <= te - 1; T += 2) {
            iter(IC<0>{}, T);
            iter(IC<1>{}, T + 1);
        }
        if (T < te - 1) {
            iter(IC<0>{}, T);
            last(IC<1>{});
        } else {
            last(IC<0>{});
        }
    }
    // normalise and store: lane holds row lrow, head-dim 32 dt + 8 (i / 4) + 4 half + i % 4
    if (!rvalid) return;
    const float lr = lsum + __shfl_xor(lsum, 32);   // both half-waves' keys
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    if (P.splits > 1) {   // a partial over tiles [tb, te): o / l, the offset m and l, in float32
        // o as [head-dim / 4][row][4] per item: column group c4 = d / 4 = 8 dt +
        // 2 q + half, so each store instruction writes two 512-byte runs
        const int64_t item_base = (int64_t)(split * P.num_work + wg) * kRows;
        const int64_t pi = item_base + wv * 32 + lrow;
        float *po = P.part + item_base * D + (wv * 32 + lrow) * 4;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c4 = 8 * dt + 2 * q + half;
                *reinterpret_cast<float4 *>(po + c4 * kRows * 4) =
                    make_float4(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv, o[dt][4 * q + 2] * inv,
                                o[dt][4 * q + 3] * inv);
            }
        if (half == 0) {
            const int64_t np = (int64_t)P.splits * P.num_work * kRows;
            P.part[np * D + pi] = lr > 0.0f ? m_used : -INFINITY;
            P.part[np * (D + 1) + pi] = lr;
        }
        return;
    }
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

// The merge of a row block's key ranges: out = sum_c w_c o_c / sum_c w_c with
// w_c = l_c 2^(m_c - M), M = max_c m_c (each o_c already divided by l_c), the
// online softmax's combination of partial results over disjoint key sets.
template <int DT, int D>
__global__ void __launch_bounds__(256) prefix_merge_kernel(const PrefixParams P) {
    constexpr int RPB = 16;   // rows per workgroup: 16 threads per column group (rows fastest, coalesced)
    const int wg = blockIdx.x / (kRows / RPB), rr = (blockIdx.x % (kRows / RPB)) * RPB + (threadIdx.x & 15);
    const int RB = P.row_blocks, KVH = P.num_kv_heads, gqa = P.gqa;
    const int s = wg / (KVH * RB), g = (wg / RB) % KVH, rb = wg % RB;
    const int q0 = P.query_start_loc[s];
    const int nrows = (P.query_start_loc[s + 1] - q0) * gqa;
    const int row = rb * kRows + rr;
    if (row >= nrows) return;
    const int64_t np = (int64_t)P.splits * P.num_work * kRows;
    float M = -INFINITY;
    for (int c = 0; c < P.splits; ++c) M = fmaxf(M, P.part[np * D + (int64_t)(c * P.num_work + wg) * kRows + rr]);
    float wc[kPrefixMaxSplits];
    float W = 0.0f;
#pragma unroll
    for (int c = 0; c < kPrefixMaxSplits; ++c) {
        wc[c] = 0.0f;
        if (c < P.splits) {
            const int64_t pi = (int64_t)(c * P.num_work + wg) * kRows + rr;
            const float l = P.part[np * (D + 1) + pi];
            if (l > 0.0f) wc[c] = l * exp2f(P.part[np * D + pi] - M);   // (a range with no visible key: 0)
            W += wc[c];
        }
    }
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    const int jq = row / gqa, rq = row - jq * gqa;
    uint8_t *orow = reinterpret_cast<uint8_t *>(P.out) + ((int64_t)(q0 + jq) * P.num_heads + g * gqa + rq) * D * 2;
#pragma unroll
    for (int k = 0; k < (D / 4 + 15) / 16; ++k) {
        const int c4 = (threadIdx.x >> 4) + 16 * k;
        if (c4 >= D / 4) break;
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
        for (int c = 0; c < kPrefixMaxSplits; ++c) {
            if (c < P.splits && wc[c] > 0.0f) {
                const int64_t ib = (int64_t)(c * P.num_work + wg) * kRows;
                const float4 v = *reinterpret_cast<const float4 *>(P.part + ib * D + ((int64_t)c4 * kRows + rr) * 4);
                a0 = fmaf(wc[c], v.x, a0);
                a1 = fmaf(wc[c], v.y, a1);
                a2 = fmaf(wc[c], v.z, a2);
                a3 = fmaf(wc[c], v.w, a3);
            }
        }
        *reinterpret_cast<u32x2 *>(orow + 8 * c4) = u32x2{pack16<DT>(a0 * inv, a1 * inv), pack16<DT>(a2 * inv, a3 * inv)};
    }
}

template <int DT, bool BUF, int D>
hipError_t launch_d(const PrefixParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)(((int64_t)p.num_work * p.splits + 7) / 8 * 8)), block(256);
    hipLaunchKernelGGL((prefix_kernel<DT, D, BUF>), grid, block, 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL((prefix_merge_kernel<DT, D>), dim3((unsigned)p.num_work * (kRows / 16)), block, 0, stream, p);
    return hipGetLastError();
}

template <int DT, bool BUF>
hipError_t launch_dt(const PrefixParams &p, int head_size, hipStream_t stream) {
    switch (head_size) {
    case 64: return launch_d<DT, BUF, 64>(p, stream);
    case 96: return launch_d<DT, BUF, 96>(p, stream);
    case 128: return launch_d<DT, BUF, 128>(p, stream);
    case 192: return launch_d<DT, BUF, 192>(p, stream);
    case 256: return launch_d<DT, BUF, 256>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

// the attention kernel of a case, for occupancy queries
const void *kernel_of(int dtype, int head_size, bool buf) {
#define PAV2_PREFIX_K(DT, D)                                                                                   \
    (buf ? reinterpret_cast<const void *>(&prefix_kernel<DT, D, true>)                                      \
         : reinterpret_cast<const void *>(&prefix_kernel<DT, D, false>))
    const bool bf = dtype == BF16;
    switch (head_size) {
    case 64: return bf ? PAV2_PREFIX_K(BF16, 64) : PAV2_PREFIX_K(F16, 64);
    case 96: return bf ? PAV2_PREFIX_K(BF16, 96) : PAV2_PREFIX_K(F16, 96);
    case 128: return bf ? PAV2_PREFIX_K(BF16, 128) : PAV2_PREFIX_K(F16, 128);
    case 192: return bf ? PAV2_PREFIX_K(BF16, 192) : PAV2_PREFIX_K(F16, 192);
    case 256: return bf ? PAV2_PREFIX_K(BF16, 256) : PAV2_PREFIX_K(F16, 256);
    default: return nullptr;
    }
#undef PAV2_PREFIX_K
}

// concurrent workgroups of a kernel on the current device (occupancy x CUs),
// queried once per (device, kernel)
int resident_slots(const void *kern) {
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kern});
    if (it != cache.end()) return it->second;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int slots = per_cu * cus;
    cache[{dev, kern}] = slots;
    return slots;
}

}  // namespace

bool prefix_mfma_supported(int dtype, int head_size, int bs_log2, float scale) {
    return (dtype == F16 || dtype == BF16) && head_size % 32 == 0 && head_size <= 256 && bs_log2 >= 3 &&
           scale > 0.0f;
}

int prefix_splits(int dtype, int head_size, bool offsets32, int num_work, int max_seq_len) {
    const void *kern = kernel_of(dtype, head_size, offsets32);
    const int slots = kern ? resident_slots(kern) : 0;
    if (slots <= 0 || num_work <= 0) return 1;
    // estimated run: rounds of resident workgroups x tiles per range, plus a
    // tile's worth for writing and merging the partials; ranges of >= 4 tiles
    const int64_t tiles = ((int64_t)max_seq_len + kKeys - 1) / kKeys;
    auto cost = [&](int sp) {
        const int64_t rounds = ((int64_t)num_work * sp + slots - 1) / slots;
        return rounds * ((tiles + sp - 1) / sp) + (sp > 1 ? 2 : 0);
    };
    int best = 1;
    for (int sp = 2; sp <= kPrefixMaxSplits && (tiles + sp - 1) / sp >= 4; ++sp)
        if (cost(sp) < cost(best)) best = sp;
    return best;
}

size_t prefix_workspace_bytes(int splits, int num_work, int head_size) {
    if (splits <= 1) return 0;
    return (size_t)splits * (size_t)num_work * kRows * (size_t)(head_size + 2) * sizeof(float);
}

hipError_t launch_prefix(const PrefixParams &p, int dtype, int head_size, hipStream_t stream) {
    if (!prefix_mfma_supported(dtype, head_size, p.bs_log2, p.scale_log2)) return hipErrorInvalidValue;
    if (p.splits < 1 || p.splits > kPrefixMaxSplits || (p.splits > 1 && !p.part)) return hipErrorInvalidValue;
    if (p.offsets32)
        return dtype == BF16 ? launch_dt<BF16, true>(p, head_size, stream) : launch_dt<F16, true>(p, head_size, stream);
    return dtype == BF16 ? launch_dt<BF16, false>(p, head_size, stream) : launch_dt<F16, false>(p, head_size, stream);
}

}  // namespace pav2
