// Phase 2 of PagedAttention V2 decode: the log-sum-exp combine of the
// per-partition results (page "paged_attention_v2_pytorch.py", the
// "Cross-partition reduction" block; page "paged_attention_v2_triton.py",
// _paged_attn_v2_reduce_kernel):
//   M = max_p m_p,  w_p = exp(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
// over the partitions p < ceil(seq_len / 512) of each (sequence, head);
// seq_len == 0 gives a zero row (page 1's zero-length branch; the page-2
// reduce would divide 0 by 0 there).  There is no cap on the partition count
// (page 2 truncates past 1024).
//
// Short contexts: one wavefront per (sequence, head), or two pairs per
// wavefront when the pairs outnumber one resident round of wavefronts; long
// contexts: 4 or 16 wavefronts per (sequence, head).  See phase2_kernel.
#include <math.h>

#include "pav2_internal.h"

namespace pav2 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// One 16-byte word of a row (4 f32 or 8 16-bit elements) as floats.
template <int ODT>
__device__ __forceinline__ void to_vec(const u32x4 w, float (&v)[ODT == F32 ? 4 : 8]) {
    if constexpr (ODT == F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = as_f32(w[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ODT == BF16) {
                v[2 * e] = as_f32(w[e] << 16);
                v[2 * e + 1] = as_f32(w[e] & 0xffff0000u);
            } else {
                f16x2 h = as_f16x2(w[e]);
                v[2 * e] = (float)h[0];
                v[2 * e + 1] = (float)h[1];
            }
        }
    }
}

template <int ODT>
__device__ __forceinline__ void store_vec(uint8_t *dst, const float (&v)[ODT == F32 ? 4 : 8]) {
    if constexpr (ODT == F32) {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ODT == BF16) {
                bf16x2 b;
                b[0] = (__bf16)v[2 * e];
                b[1] = (__bf16)v[2 * e + 1];
                w[e] = __builtin_bit_cast(uint32_t, b);
            } else {
                f16x2 b;
                b[0] = (_Float16)v[2 * e];
                b[1] = (_Float16)v[2 * e + 1];
                w[e] = __builtin_bit_cast(uint32_t, b);
            }
        }
        *reinterpret_cast<u32x4 *>(dst) = w;
    }
}

// Online (max, sum of exp-weighted exp_sums) pair combine.
__device__ __forceinline__ void lse_merge(float &m, float &w, float m2, float w2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;   // both empty
    w = w * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + w2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
    m = mn;
}

// WPP wavefronts per (sequence, head): 1 for short contexts (a workgroup
// serves 4 pairs, or 8 with PPW = 2 pairs per wavefront, 32 lanes each), 4 or
// 16 for long ones (one pair per workgroup).  A pair's LPP = 64 / PPW lanes
// form G groups of TPR lanes; lane (gi, r) owns VEC consecutive head-dim
// elements r*VEC.. of the row and the partitions q, q + Q, q + 2Q, ... with
// q = sub*G + gi and Q = WPP*G groups in all.
//   1. One pass over the used partitions' statistics gives the global
//      (max M, sum W of exp(m_p - M) l_p) by an online merge; the first batch
//      of tmp_output rows is loaded alongside it.
//   2. Each lane accumulates exp(m_p - M) l_p * o_p over its partitions.
//   3. Groups are added across lanes, then (WPP = 4) across wavefronts in LDS;
//      the row is scaled by 1 / W and stored.
template <int ODT, int D, int WPP, int PPW>
__global__ void __launch_bounds__(64 * (WPP > 4 ? WPP : 4))
__attribute__((amdgpu_waves_per_eu(PPW == 2 ? 4 : 1))) phase2_kernel(const Phase2Params P) {
    static_assert(PPW == 1 || (PPW == 2 && WPP == 1), "two pairs per wavefront: short contexts only");
    constexpr int VEC = ODT == F32 ? 4 : 8;
    constexpr int EB = ODT == F32 ? 4 : 2;
    constexpr int LPP = 64 / PPW;                   // lanes per pair
    constexpr int TPR = D / VEC;                    // lanes per row
    constexpr int G = LPP / TPR;                    // partition groups per pair and wavefront
    constexpr int Q = WPP * G;                      // partition groups per pair
    constexpr int B = WPP == 4 ? 16 : (PPW == 2 ? 12 : 8);   // rows in flight per lane
    constexpr int WG_WAVES = WPP > 4 ? WPP : 4;
    static_assert(D % VEC == 0 && TPR <= LPP, "row split");
    __shared__ float red[WPP > 1 ? WPP * D : 1];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * WG_WAVES + wv;
    const int pb = PPW == 2 ? (lane & 32) : 0;     // the pair's first lane in the wavefront
    const int pl = lane - pb;                       // lane within the pair
    const int64_t sh = PPW == 2 ? gw * 2 + (pb >> 5) : gw / WPP;   // s * H + h
    const int sub = (int)(gw % WPP);
    // past the last pair: uniform per workgroup when WPP > 1, per pair (both
    // halves of a wavefront are then done) when PPW = 2
    if (sh >= (int64_t)P.num_seqs * P.num_heads) return;
    const int s = (int)(sh / P.num_heads);
    const int maxP = P.max_num_partitions;
    const int L = P.seq_lens[s];
    int np = (L + kPartition - 1) / kPartition;
    np = np < maxP ? np : maxP;
    const int gi = pl / TPR;
    const int r = pl - gi * TPR;
    const bool active = gi < G;
    const int q = sub * G + gi;
    uint8_t *out = reinterpret_cast<uint8_t *>(P.out) + (sh * D + r * VEC) * EB;

    if (L <= 0) {
        if (sub == 0 && gi == 0) {
            float z[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) z[e] = 0.0f;
            store_vec<ODT>(out, z);
        }
        return;
    }

    const float *ml = P.max_logits + sh * maxP;
    const float *es = P.exp_sums + sh * maxP;
    const uint8_t *src = reinterpret_cast<const uint8_t *>(P.tmp_out) + (sh * maxP * D + r * VEC) * EB;

    // A batch: B rows of this lane with their statistics, loaded together;
    // the rows stay as loaded (16-byte words) until they are accumulated.
    u32x4 v[B];
    float bm[B], be[B];
    auto load_batch = [&](int p0) {
#pragma unroll
        for (int k = 0; k < B; ++k) {
            const int p = p0 + k * Q;
            bm[k] = -INFINITY;
            be[k] = 0.0f;
            if (active && p < np) {
                v[k] = *reinterpret_cast<const u32x4 *>(src + (int64_t)p * D * EB);
                bm[k] = ml[p];
                be[k] = es[p];
            }
        }
    };
    load_batch(q);   // the first batch is in flight during the statistics pass

    float m = -INFINITY, w = 0.0f;
    for (int p0 = pl; p0 < np; p0 += 4 * LPP) {
        float sm[4], se[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int p = p0 + k * LPP;
            sm[k] = p < np ? ml[p] : -INFINITY;
            se[k] = p < np ? es[p] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) lse_merge(m, w, sm[k], se[k]);
    }
#pragma unroll
    for (int off = LPP / 2; off > 0; off >>= 1) {   // within the pair's lanes
        const float m2 = __shfl_xor(m, off), w2 = __shfl_xor(w, off);
        lse_merge(m, w, m2, w2);
    }

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    auto add_batch = [&]() {
#pragma unroll
        for (int k = 0; k < B; ++k) {
            if (be[k] != 0.0f) {   // rows past np (and inactive lanes) carry be = 0
                const float wp = __builtin_amdgcn_exp2f((bm[k] - m) * kLog2e) * be[k];
                float x[VEC];
                to_vec<ODT>(v[k], x);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] += wp * x[e];
            }
        }
    };
    add_batch();
    for (int p0 = q + B * Q; p0 < np; p0 += B * Q) {
        load_batch(p0);
        add_batch();
    }
    // add the pair's G groups (lanes r, r + TPR, ... of the pair)
    if constexpr ((G & (G - 1)) == 0 && G * TPR == LPP) {
#pragma unroll
        for (int off = TPR; off < LPP; off <<= 1)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
    } else {
        float t[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) t[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < G; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) t[e] += __shfl(acc[e], pb + r + k * TPR);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = t[e];
    }
    if constexpr (WPP > 1) {
        if (gi == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) red[sub * D + r * VEC + e] = acc[e];
        }
        __syncthreads();
        if (sub != 0) return;
        if (gi == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float a = 0.0f;
#pragma unroll
                for (int k = 0; k < WPP; ++k) a += red[k * D + r * VEC + e];
                acc[e] = a;
            }
        }
    }
    if (gi == 0) {
        // w == 0: every partition empty (block-sparse heads that attend
        // no token): a zero row, as for an empty sequence
        const float inv = w > 0.0f ? 1.0f / w : 0.0f;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = acc[e] * inv;
        store_vec<ODT>(out, o);
    }
}

template <int ODT, int D, int WPP, int PPW>
hipError_t launch_wpp(const Phase2Params &p, hipStream_t stream) {
    constexpr int WG_WAVES = WPP > 4 ? WPP : 4;
    const int64_t pairs = (int64_t)p.num_seqs * p.num_heads;
    const int64_t waves = (pairs + PPW - 1) / PPW * WPP;
    const dim3 grid((unsigned)((waves + WG_WAVES - 1) / WG_WAVES));
    hipLaunchKernelGGL((phase2_kernel<ODT, D, WPP, PPW>), grid, dim3(64 * WG_WAVES), 0, stream, p);
    return hipGetLastError();
}

template <int ODT, int D>
hipError_t launch_one(const Phase2Params &p, hipStream_t stream) {
    switch (phase2_waves_per_pair(p.max_num_partitions)) {
    case 16: return launch_wpp<ODT, D, 16, 1>(p, stream);
    case 4: return launch_wpp<ODT, D, 4, 1>(p, stream);
    default:
        if constexpr (D / (ODT == F32 ? 4 : 8) <= 32) {
            if (phase2_pairs_per_wave((int64_t)p.num_seqs * p.num_heads, p.max_num_partitions, D, ODT) == 2)
                return launch_wpp<ODT, D, 1, 2>(p, stream);
        }
        return launch_wpp<ODT, D, 1, 1>(p, stream);
    }
}

template <int ODT>
hipError_t launch_d(const Phase2Params &p, int D, int lds, hipStream_t stream) {
    (void)lds;
    switch (D) {
    case 64: return launch_one<ODT, 64>(p, stream);
    case 80: return launch_one<ODT, 80>(p, stream);
    case 96: return launch_one<ODT, 96>(p, stream);
    case 112: return launch_one<ODT, 112>(p, stream);
    case 120: return launch_one<ODT, 120>(p, stream);
    case 128: return launch_one<ODT, 128>(p, stream);
    case 192: return launch_one<ODT, 192>(p, stream);
    case 256: return launch_one<ODT, 256>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

// ---- device-side decoding of KV elements (test hook) -------------------------

template <int KVDT, int VIA>
__global__ void decode_kv_kernel(const uint8_t *src, float *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if constexpr (KVDT == F32) {
        dst[i] = reinterpret_cast<const float *>(src)[i];
    } else if constexpr (KVDT == F16) {
        dst[i] = (float)reinterpret_cast<const _Float16 *>(src)[i];
    } else if constexpr (KVDT == BF16) {
        dst[i] = as_f32((uint32_t)reinterpret_cast<const uint16_t *>(src)[i] << 16);
    } else {
        // the same converters the phase-1 kernel applies to an e4m3 byte
        const uint32_t w = src[i];
        if constexpr (VIA == F32) {
            dst[i] = __builtin_amdgcn_cvt_pk_f32_fp8(w, false)[0];
        } else if constexpr (VIA == BF16) {
            const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
            dst[i] = as_f32(b << 16);
        } else {
            const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
            dst[i] = (float)as_f16x2(b)[0];
        }
    }
}

}  // namespace

hipError_t launch_phase2(const Phase2Params &p, int odt, int head_size, int threads, int lds_bytes,
                         hipStream_t stream) {
    if (threads != kPhase2Threads) return hipErrorInvalidValue;
    switch (odt) {
    case F32: return launch_d<F32>(p, head_size, lds_bytes, stream);
    case F16: return launch_d<F16>(p, head_size, lds_bytes, stream);
    case BF16: return launch_d<BF16>(p, head_size, lds_bytes, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_kv(const void *src, float *dst, int64_t n, int dtype, int via,
                            hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    const uint8_t *s = reinterpret_cast<const uint8_t *>(src);
    switch (dtype) {
    case F32: hipLaunchKernelGGL((decode_kv_kernel<F32, F32>), grid, dim3(256), 0, stream, s, dst, n); break;
    case F16: hipLaunchKernelGGL((decode_kv_kernel<F16, F16>), grid, dim3(256), 0, stream, s, dst, n); break;
    case BF16: hipLaunchKernelGGL((decode_kv_kernel<BF16, BF16>), grid, dim3(256), 0, stream, s, dst, n); break;
    case FP8:
        if (via == F32) hipLaunchKernelGGL((decode_kv_kernel<FP8, F32>), grid, dim3(256), 0, stream, s, dst, n);
        else if (via == BF16) hipLaunchKernelGGL((decode_kv_kernel<FP8, BF16>), grid, dim3(256), 0, stream, s, dst, n);
        else if (via == F16) hipLaunchKernelGGL((decode_kv_kernel<FP8, F16>), grid, dim3(256), 0, stream, s, dst, n);
        else return hipErrorInvalidValue;
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pav2
