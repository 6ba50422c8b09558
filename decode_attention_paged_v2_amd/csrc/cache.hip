// KV-cache write on gfx950: the new tokens' keys and values enter the paged
// caches through a slot mapping (page "paged_attn.py", write_to_paged_cache,
// which calls reshape_and_cache; cache layouts from split_kv_cache on the
// same page).  Token t goes to slot s = slot_mapping[t], i.e. block s / bs,
// offset s % bs:
//
//   key_cache  [blk, g, i / x, off, i % x] = enc(key  [t, g, i] / k_scale)
//   value_cache[blk, g, i,     off]        = enc(value[t, g, i] / v_scale)
//
// with x = 16 / element size of the cache dtype.  The quotient is the IEEE
// float32 quotient (see quotient()); enc rounds it to the cache dtype to
// nearest, ties to even (e4m3 after saturating to +-448, so no value
// overflows to NaN).  With unit scales and a cache of the input's dtype the
// write is a plain copy.  Slots < 0, or past the pool, write nothing.
//
// One workgroup per (tile of consecutive tokens, kv head): 16 tokens, or 32
// for one-byte caches so that a prefill tile fills whole 32-byte value rows
// of a 32-token block (a half-written row would leave each 64-byte line to
// two workgroups).  The tile moves through LDS in both directions:
//
// * loads: lanes take consecutive 16-byte vectors of the tile's token rows
//   (a token's row for one kv head is d contiguous elements), so every
//   wavefront reads whole lines; each vector is converted to the cache dtype
//   and written to LDS -- keys in cache order as 16-byte cache vectors
//   [chunk][token], values as converted token rows [token][head dim] (rows
//   padded by 16 bytes, so neither the row writes nor the column reads below
//   conflict in LDS banks);
// * stores: keys token-fastest (tokens with consecutive slots give
//   block_size * 16 contiguous bytes per chunk); values as 8 tokens of one
//   head-dim row per lane (gathered from the 8 token rows in LDS), one
//   vector store when their slots are 8 consecutive, 8-aligned positions in
//   a block of at least 8 tokens (then always within one block, as block
//   sizes are powers of two), else element by element.
#include "cache.h"

namespace pav2 {
namespace {

constexpr int kCacheThreads = 256;
constexpr int kMaxHead = 256;

template <int DT>
constexpr int esize() { return DT == F32 ? 4 : (DT == FP8 ? 1 : 2); }

template <int CDT>
constexpr int tile_tokens() { return esize<CDT>() == 1 ? 32 : 16; }

// Element e of a run of 32-bit words holding elements of dtype DT, as float.
template <int DT>
__device__ __forceinline__ float widen(const uint32_t *w, int e) {
    if constexpr (DT == F32) return as_f32(w[e]);
    else if constexpr (DT == BF16) return as_f32((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
    else {
        const f16x2 h = as_f16x2(w[e >> 1]);
        return (float)((e & 1) ? h[1] : h[0]);
    }
}

__device__ __forceinline__ float sat_e4m3(float f) {
    // comparisons with NaN are false, so NaN passes through unchanged
    return f > 448.0f ? 448.0f : (f < -448.0f ? -448.0f : f);
}

// N floats (N a multiple of 4) -> N elements of dtype DT packed in words.
template <int DT, int N>
__device__ __forceinline__ void encode(const float (&f)[N], uint32_t (&w)[N * esize<DT>() / 4]) {
    if constexpr (DT == F32) {
#pragma unroll
        for (int e = 0; e < N; ++e) w[e] = as_u32(f[e]);
    } else if constexpr (DT == FP8) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(f[4 * k]), sat_e4m3(f[4 * k + 1]), 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(f[4 * k + 2]), sat_e4m3(f[4 * k + 3]), v, true);
            w[k] = (uint32_t)v;
        }
    } else if constexpr (DT == BF16) {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            bf16x2 v;
            v[0] = (__bf16)f[2 * k];
            v[1] = (__bf16)f[2 * k + 1];
            w[k] = __builtin_bit_cast(uint32_t, v);
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            f16x2 v;
            v[0] = (_Float16)f[2 * k];
            v[1] = (_Float16)f[2 * k + 1];
            w[k] = __builtin_bit_cast(uint32_t, v);
        }
    }
}

// a / b rounded to nearest (IEEE float32 division), given y = RN(1 / b).
// Fast path (Markstein's correction): q = RN(a * y) is within one ulp of
// a / b, the residual a - b * q is exact in one FMA, and RN(q + r * y) is the
// correctly rounded quotient -- valid while a, q and the residual stay well
// inside the normal range (checked per element) and y is normal (checked on
// the host, `fast`).  Everything else takes the division itself.
__device__ __forceinline__ float quotient(float a, float b, float y, bool fast) {
    const float q = a * y;
    const float aq = fabsf(q), aa = fabsf(a);
    if (fast && aq >= 0x1p-100f && aq <= 0x1p100f && aa >= 0x1p-96f && aa <= 0x1p100f)
        return fmaf(fmaf(-q, b, a), y, q);
    return a / b;
}

// One 16-byte input vector (16 / sizeof(input) elements) -> the same
// elements in the cache dtype, packed in words.
template <int IDT, int CDT, bool SCALED>
__device__ __forceinline__ void convert16(const u32x4 v, float scale, float rcp, bool fast,
                                          uint32_t (&out)[(16 / esize<IDT>()) * esize<CDT>() / 4]) {
    constexpr int N = 16 / esize<IDT>();
    const uint32_t in[4] = {v[0], v[1], v[2], v[3]};
    if constexpr (IDT == CDT && !SCALED) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = in[k];   // x / 1 rounds to x: copy the bits
    } else {
        float f[N];
#pragma unroll
        for (int e = 0; e < N; ++e) {
            f[e] = widen<IDT>(in, e);
            if constexpr (SCALED) f[e] = quotient(f[e], scale, rcp, fast);
        }
        encode<CDT, N>(f, out);
    }
}

template <int NW>
__device__ __forceinline__ void store_words(uint8_t *dst, const uint32_t *w) {
    if constexpr (NW == 2) {
        __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2 *>(dst));
    } else {
#pragma unroll
        for (int k = 0; k < NW / 4; ++k)
            __builtin_nontemporal_store(u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]},
                                        reinterpret_cast<u32x4 *>(dst) + k);
    }
}

template <int IDT, int CDT, int D, bool SCALED>
__global__ void __launch_bounds__(kCacheThreads) cache_write_kernel(const CacheParams P) {
    constexpr int IB = esize<IDT>();
    constexpr int CB = esize<CDT>();
    constexpr int X = 16 / CB;            // elements per 16-byte cache vector (keys)
    constexpr int EV = 16 / IB;           // elements per 16-byte input vector
    constexpr int NV = D / EV;            // input vectors per token row
    constexpr int NC = D / X;             // cache vectors (key chunks) per token
    constexpr int TT = tile_tokens<CDT>();
    constexpr int NG = TT / 8;            // 8-token value groups per tile
    constexpr int SK = TT * 16 + 16;      // LDS bytes per key chunk row (padded)
    constexpr int RV = D * CB + 16;       // LDS bytes per converted value token row (padded)
    __shared__ __align__(16) uint8_t s_k[NC * SK];
    __shared__ __align__(16) uint8_t s_v[TT * RV];
    __shared__ int64_t s_slot[TT];

    const int tid = threadIdx.x;
    const int g = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * TT;
    const int bs_log2 = P.bs_log2;
    const int64_t bs_mask = (1 << bs_log2) - 1;
    const int64_t row_in = (int64_t)P.num_kv_heads * D * IB;   // input bytes per token
    const int ntok = (int)min((int64_t)TT, P.num_tokens - t0);

    if (tid < TT) {
        int64_t sl = -1;
        if (tid < ntok) sl = P.slot_mapping[t0 + tid];
        s_slot[tid] = (sl >= 0 && sl < P.num_slots) ? sl : -1;
    }

    // loads: keys (vectors [0, TT * NV)), then values; consecutive lanes take
    // consecutive vectors of a token row
    const uint8_t *kin = P.key + t0 * row_in + (int64_t)g * D * IB;
    const uint8_t *vin = P.value + t0 * row_in + (int64_t)g * D * IB;
    constexpr int OW = EV * CB / 4;       // cache words per input vector
    for (int v = tid; v < 2 * TT * NV; v += kCacheThreads) {
        const bool is_v = v >= TT * NV;
        const int u = is_v ? v - TT * NV : v;
        const int t = u / NV, k = u - t * NV;
        if (t >= ntok) continue;
        const uint8_t *src = (is_v ? vin : kin) + t * row_in + k * 16;
        const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
        uint32_t w[OW > 0 ? OW : 1];
        convert16<IDT, CDT, SCALED>(raw, is_v ? P.v_scale : P.k_scale, is_v ? P.v_rcp : P.k_rcp,
                                    P.fast_div != 0, w);
        // keys: elements k*EV .. k*EV+EV-1 lie in key chunk k / (X/EV);
        // values: the same bytes of the token's converted row
        uint8_t *dst = is_v ? s_v + t * RV + k * EV * CB
                            : s_k + (k / (X / EV)) * SK + t * 16 + (k % (X / EV)) * EV * CB;
        if constexpr (OW == 4) *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        else if constexpr (OW == 2) *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
        else *reinterpret_cast<uint32_t *>(dst) = w[0];
    }
    __syncthreads();

    const int64_t head_off = (int64_t)g * P.head_stride;

    // keys: one 16-byte cache vector per lane, tokens fastest
    for (int idx = tid; idx < NC * TT; idx += kCacheThreads) {
        const int t = idx % TT, c = idx / TT;
        const int64_t sl = s_slot[t];
        if (sl < 0) continue;
        const u32x4 w = *reinterpret_cast<const u32x4 *>(s_k + c * SK + t * 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(P.key_cache + (sl >> bs_log2) * P.blk_stride +
                                                                  head_off + (((int64_t)c << bs_log2) + (sl & bs_mask)) * 16));
    }

    // values: 8 tokens of one head-dim row per lane
    {
        const int h = tid % NG;
        int64_t sl[8];
        bool run = true;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            sl[k] = s_slot[8 * h + k];
            run = run && sl[k] >= 0 && sl[k] == sl[0] + k;
        }
        run = run && (sl[0] & 7) == 0 && bs_log2 >= 3;   // 8 aligned slots share one block of >= 8
        uint8_t *vbase = P.value_cache + head_off;
        for (int i = tid / NG; i < D; i += kCacheThreads / NG) {
            // element i of tokens 8h .. 8h+7, packed in words
            uint32_t w[8 * CB / 4];
#pragma unroll
            for (int k = 0; k < 8 * CB / 4; ++k) w[k] = 0u;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint8_t *src = s_v + (8 * h + k) * RV + i * CB;
                if constexpr (CB == 4) w[k] = *reinterpret_cast<const uint32_t *>(src);
                else if constexpr (CB == 2) w[k >> 1] |= (uint32_t)*reinterpret_cast<const uint16_t *>(src) << (16 * (k & 1));
                else w[k >> 2] |= (uint32_t)*src << (8 * (k & 3));
            }
            if (run) {
                store_words<8 * CB / 4>(vbase + (sl[0] >> bs_log2) * P.blk_stride +
                                            (((int64_t)i << bs_log2) + (sl[0] & bs_mask)) * CB, w);
            } else {
                const uint8_t *wb = reinterpret_cast<const uint8_t *>(w);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (sl[k] < 0) continue;
                    uint8_t *dst = vbase + (sl[k] >> bs_log2) * P.blk_stride +
                                   (((int64_t)i << bs_log2) + (sl[k] & bs_mask)) * CB;
                    if constexpr (CB == 4) *reinterpret_cast<uint32_t *>(dst) = w[k];
                    else if constexpr (CB == 2) *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
                    else *dst = wb[k];
                }
            }
        }
    }
}

template <int IDT, int CDT, int D>
hipError_t launch_d(const CacheParams &p, bool scaled, hipStream_t stream) {
    constexpr int TT = tile_tokens<CDT>();
    const dim3 grid((unsigned)((p.num_tokens + TT - 1) / TT), (unsigned)p.num_kv_heads);
    if (scaled)
        hipLaunchKernelGGL((cache_write_kernel<IDT, CDT, D, true>), grid, dim3(kCacheThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((cache_write_kernel<IDT, CDT, D, false>), grid, dim3(kCacheThreads), 0, stream, p);
    return hipGetLastError();
}

template <int IDT, int CDT>
hipError_t launch_scaled(const CacheParams &p, bool scaled, hipStream_t stream) {
    switch (p.head_size) {
    case 64: return launch_d<IDT, CDT, 64>(p, scaled, stream);
    case 80: return launch_d<IDT, CDT, 80>(p, scaled, stream);
    case 96: return launch_d<IDT, CDT, 96>(p, scaled, stream);
    case 112: return launch_d<IDT, CDT, 112>(p, scaled, stream);
    case 128: return launch_d<IDT, CDT, 128>(p, scaled, stream);
    case 192: return launch_d<IDT, CDT, 192>(p, scaled, stream);
    case 256: return launch_d<IDT, CDT, 256>(p, scaled, stream);
    case 120:
        if constexpr (CDT != FP8) return launch_d<IDT, CDT, 120>(p, scaled, stream);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int IDT>
hipError_t launch_cdt(const CacheParams &p, int cdt, bool scaled, hipStream_t stream) {
    if (cdt == IDT) return launch_scaled<IDT, IDT>(p, scaled, stream);
    if (cdt == FP8) return launch_scaled<IDT, FP8>(p, scaled, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cache_write(const CacheParams &p, int idt, int cdt, hipStream_t stream) {
    if (p.num_tokens == 0) return hipSuccess;
    if (p.head_size > kMaxHead || p.head_size % 8 != 0 || (cdt == FP8 && p.head_size % 16 != 0))
        return hipErrorInvalidValue;
    const bool scaled = !(p.k_scale == 1.0f && p.v_scale == 1.0f);
    switch (idt) {
    case F32: return launch_cdt<F32>(p, cdt, scaled, stream);
    case F16: return launch_cdt<F16>(p, cdt, scaled, stream);
    case BF16: return launch_cdt<BF16>(p, cdt, scaled, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pav2
