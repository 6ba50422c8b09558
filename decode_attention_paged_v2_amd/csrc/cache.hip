// KV-cache write on gfx950: the new tokens' keys and values enter the paged
// caches through a slot mapping (page "paged_attn.py", write_to_paged_cache,
// which calls reshape_and_cache; cache layouts from split_kv_cache on the
// same page).  Token t goes to slot s = slot_mapping[t], i.e. block s / bs,
// offset s % bs:
//
//   key_cache  [blk, g, i / x, off, i % x] = enc(key  [t, g, i] / k_scale)
//   value_cache[blk, g, i,     off]        = enc(value[t, g, i] / v_scale)
//
// with x = 16 / element size of the cache dtype.  The quotient is an IEEE
// float32 division; enc rounds to the cache dtype to nearest, ties to even
// (e4m3 after saturating to +-448, so no value overflows to NaN).  With unit
// scales and a cache of the input's dtype the write is a plain copy.  Slots
// < 0, or past the pool, write nothing.
//
// One workgroup per (16 consecutive tokens, kv head).  Keys: a lane converts
// one 16-byte cache vector (x elements of one token) and stores it; lanes are
// token-fastest, so tokens with consecutive slots give contiguous stores, and
// the four vectors a wavefront takes from one token are 64 contiguous input
// bytes.  Values: a token's head-dim row must be scattered over d cache rows
// of block_size elements, so the tile is transposed through LDS; each lane
// then stores 8 tokens of one head-dim row as one vector when their slots are
// 8 consecutive, 8-aligned positions (always within one block, as block sizes
// are powers of two >= 8), else element by element.
#include "pav2_internal.h"

namespace pav2 {
namespace {

constexpr int kTileTokens = 16;
constexpr int kCacheThreads = 256;
constexpr int kMaxHead = 256;

template <int DT>
constexpr int esize() { return DT == F32 ? 4 : (DT == FP8 ? 1 : 2); }

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

// N input elements at `src` (16-byte aligned) -> N cache elements in words.
template <int IDT, int CDT, bool SCALED, int N>
__device__ __forceinline__ void convert(const uint8_t *src, float scale, uint32_t (&out)[N * esize<CDT>() / 4]) {
    constexpr int IW = N * esize<IDT>() / 4;   // input words
    uint32_t in[IW];
#pragma unroll
    for (int k = 0; k < IW / 4; ++k) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src) + k);
        in[4 * k + 0] = v[0];
        in[4 * k + 1] = v[1];
        in[4 * k + 2] = v[2];
        in[4 * k + 3] = v[3];
    }
    if constexpr (IDT == CDT && !SCALED) {
#pragma unroll
        for (int k = 0; k < IW; ++k) out[k] = in[k];   // x / 1 rounds to x: copy the bits
    } else {
        float f[N];
#pragma unroll
        for (int e = 0; e < N; ++e) {
            f[e] = widen<IDT>(in, e);
            if constexpr (SCALED) f[e] = f[e] / scale;
        }
        encode<CDT, N>(f, out);
    }
}

template <int NW>
__device__ __forceinline__ void store_words(uint8_t *dst, const uint32_t (&w)[NW]) {
    if constexpr (NW == 2) {
        __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2 *>(dst));
    } else {
#pragma unroll
        for (int k = 0; k < NW / 4; ++k)
            __builtin_nontemporal_store(u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]},
                                        reinterpret_cast<u32x4 *>(dst) + k);
    }
}

template <int IDT, int CDT, bool SCALED>
__global__ void __launch_bounds__(kCacheThreads) cache_write_kernel(const CacheParams P) {
    constexpr int IB = esize<IDT>();
    constexpr int CB = esize<CDT>();
    constexpr int X = 16 / CB;            // elements per 16-byte key vector
    constexpr int RS = kTileTokens * CB + 16;   // LDS row stride (bytes) of the transposed values
    __shared__ __align__(16) uint8_t s_v[kMaxHead * RS];
    __shared__ int64_t s_slot[kTileTokens];

    const int tid = threadIdx.x;
    const int t = tid & (kTileTokens - 1);
    const int j = tid >> 4;
    const int g = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * kTileTokens;
    const int D = P.head_size;
    const int bs_log2 = P.bs_log2;
    const int64_t bs_mask = (1 << bs_log2) - 1;
    const int64_t row_in = (int64_t)P.num_kv_heads * D * IB;   // input bytes per token

    if (tid < kTileTokens) {
        int64_t sl = -1;
        if (t0 + tid < P.num_tokens) sl = P.slot_mapping[t0 + tid];
        s_slot[tid] = (sl >= 0 && sl < P.num_slots) ? sl : -1;
    }

    // values: 8 head-dim elements of token t per step, transposed into LDS
    const bool tok_ok = t0 + t < P.num_tokens;
    const uint8_t *vin = P.value + (t0 + t) * row_in + (int64_t)g * D * IB;
    for (int c = j; c < D / 8; c += kCacheThreads / kTileTokens) {
        uint32_t w[8 * CB / 4 > 0 ? 8 * CB / 4 : 1];
        if (tok_ok) {
            convert<IDT, CDT, SCALED, 8>(vin + c * 8 * IB, P.v_scale, w);
        } else {
#pragma unroll
            for (int k = 0; k < 8 * CB / 4; ++k) w[k] = 0u;
        }
        const uint8_t *wb = reinterpret_cast<const uint8_t *>(w);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint8_t *dst = s_v + (8 * c + k) * RS + t * CB;
            if constexpr (CB == 4) *reinterpret_cast<uint32_t *>(dst) = w[k];
            else if constexpr (CB == 2) *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
            else *dst = wb[k];
        }
    }
    __syncthreads();

    const int64_t head_off = (int64_t)g * P.head_stride;

    // keys: one 16-byte cache vector (x elements) per lane and step
    {
        const int64_t sl = s_slot[t];
        if (sl >= 0) {
            const uint8_t *kin = P.key + (t0 + t) * row_in + (int64_t)g * D * IB;
            uint8_t *kout = P.key_cache + (sl >> bs_log2) * P.blk_stride + head_off + (sl & bs_mask) * 16;
            const int nc = D / X;
            for (int c = j; c < nc; c += kCacheThreads / kTileTokens) {
                uint32_t w[4];
                convert<IDT, CDT, SCALED, X>(kin + c * X * IB, P.k_scale, w);
                store_words<4>(kout + ((int64_t)c << (bs_log2 + 4)), w);
            }
        }
    }

    // values: 8 tokens of one head-dim row per lane and step
    {
        const int h = tid & 1;
        int64_t sl[8];
        bool run = true;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            sl[k] = s_slot[8 * h + k];
            run = run && sl[k] >= 0 && sl[k] == sl[0] + k;
        }
        run = run && (sl[0] & 7) == 0;
        uint8_t *vbase = P.value_cache + head_off;
        for (int i = tid >> 1; i < D; i += kCacheThreads / 2) {
            const uint8_t *src = s_v + i * RS + 8 * h * CB;
            if (run) {
                uint32_t w[8 * CB / 4];
#pragma unroll
                for (int k = 0; k < 8 * CB / 4; ++k) w[k] = reinterpret_cast<const uint32_t *>(src)[k];
                store_words<8 * CB / 4>(vbase + (sl[0] >> bs_log2) * P.blk_stride +
                                            (((int64_t)i << bs_log2) + (sl[0] & bs_mask)) * CB, w);
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (sl[k] < 0) continue;
                    uint8_t *dst = vbase + (sl[k] >> bs_log2) * P.blk_stride +
                                   (((int64_t)i << bs_log2) + (sl[k] & bs_mask)) * CB;
                    if constexpr (CB == 4) *reinterpret_cast<uint32_t *>(dst) = reinterpret_cast<const uint32_t *>(src)[k];
                    else if constexpr (CB == 2) *reinterpret_cast<uint16_t *>(dst) = reinterpret_cast<const uint16_t *>(src)[k];
                    else *dst = src[k];
                }
            }
        }
    }
}

template <int IDT, int CDT>
hipError_t launch_scaled(const CacheParams &p, bool scaled, hipStream_t stream) {
    const dim3 grid((unsigned)((p.num_tokens + kTileTokens - 1) / kTileTokens), (unsigned)p.num_kv_heads);
    if (scaled)
        hipLaunchKernelGGL((cache_write_kernel<IDT, CDT, true>), grid, dim3(kCacheThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((cache_write_kernel<IDT, CDT, false>), grid, dim3(kCacheThreads), 0, stream, p);
    return hipGetLastError();
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
