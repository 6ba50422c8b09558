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
// One workgroup per (sequence, head).  Weights are computed once into LDS;
// the partitions are then split across thread groups, each thread reading one
// 16-byte vector of a partition row per step (rows are contiguous in
// tmp_output), and the groups' partial sums are added through LDS.
#include <math.h>

#include "pav2_internal.h"

namespace pav2 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float block_reduce(float v, float *scratch, bool is_max) {
    for (int off = 32; off > 0; off >>= 1) {
        float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int wv = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[wv] = v;
    __syncthreads();
    v = scratch[0];
    for (int i = 1; i < nw; ++i) v = is_max ? fmaxf(v, scratch[i]) : v + scratch[i];
    return v;
}

template <int ODT>
__device__ __forceinline__ void load_vec(const uint8_t *src, float (&v)[ODT == F32 ? 4 : 8]) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
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

template <int ODT, int D>
__global__ void __launch_bounds__(kPhase2Threads) phase2_kernel(const Phase2Params P) {
    constexpr int VEC = ODT == F32 ? 4 : 8;
    constexpr int EB = ODT == F32 ? 4 : 2;
    constexpr int TPR = D / VEC;                    // threads per partition row
    constexpr int G = kPhase2Threads / TPR;         // partition groups
    extern __shared__ __align__(16) float sm[];

    const int maxP = P.max_num_partitions;
    float *s_w = sm;                                // [maxP] combine weights
    float *s_red = sm + maxP;                       // [G][D] partial sums
    float *s_misc = s_red + G * D;                  // [64] reduction scratch

    const int tid = threadIdx.x;
    const int64_t sh = blockIdx.x;                  // s * H + h
    const int s = (int)(sh / P.num_heads);
    const int L = P.seq_lens[s];
    int np = (L + kPartition - 1) / kPartition;
    np = np < maxP ? np : maxP;
    uint8_t *out = reinterpret_cast<uint8_t *>(P.out) + sh * D * EB;

    if (L <= 0) {
        if (tid < TPR) {
            float z[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) z[e] = 0.0f;
            store_vec<ODT>(out + tid * VEC * EB, z);
        }
        return;
    }

    const float *ml = P.max_logits + sh * maxP;
    const float *es = P.exp_sums + sh * maxP;
    float mx = -INFINITY;
    for (int p = tid; p < np; p += kPhase2Threads) mx = fmaxf(mx, ml[p]);
    const float M = block_reduce(mx, s_misc, true);
    float ws = 0.0f;
    for (int p = tid; p < np; p += kPhase2Threads) {
        const float w = __builtin_amdgcn_exp2f((ml[p] - M) * kLog2e) * es[p];
        s_w[p] = w;
        ws += w;
    }
    const float W = block_reduce(ws, s_misc + 8, false);   // its barriers publish s_w

    const int r = tid % TPR;
    const int gi = tid / TPR;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    if (gi < G) {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(P.tmp_out) +
                             (sh * maxP * D + r * VEC) * EB;
        int p = gi;
        for (; p + 3 * G < np; p += 4 * G) {
            float v0[VEC], v1[VEC], v2[VEC], v3[VEC];
            load_vec<ODT>(src + (int64_t)p * D * EB, v0);
            load_vec<ODT>(src + (int64_t)(p + G) * D * EB, v1);
            load_vec<ODT>(src + (int64_t)(p + 2 * G) * D * EB, v2);
            load_vec<ODT>(src + (int64_t)(p + 3 * G) * D * EB, v3);
            const float w0 = s_w[p], w1 = s_w[p + G], w2 = s_w[p + 2 * G], w3 = s_w[p + 3 * G];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += w0 * v0[e] + w1 * v1[e] + w2 * v2[e] + w3 * v3[e];
        }
        for (; p < np; p += G) {
            float v0[VEC];
            load_vec<ODT>(src + (int64_t)p * D * EB, v0);
            const float w0 = s_w[p];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += w0 * v0[e];
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_red[gi * D + r * VEC + e] = acc[e];
    }
    __syncthreads();
    if (tid < TPR) {
        float v[VEC];
        const float inv = 1.0f / W;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float a = 0.0f;
            for (int k = 0; k < G; ++k) a += s_red[k * D + tid * VEC + e];
            v[e] = a * inv;
        }
        store_vec<ODT>(out + tid * VEC * EB, v);
    }
}

template <int ODT>
hipError_t launch_d(const Phase2Params &p, int D, int lds, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.num_seqs * p.num_heads));
    const dim3 block(kPhase2Threads);
#define PAV2_P2(DD)                                                                        \
    case DD:                                                                               \
        if (lds > 65536)                                                                   \
            hipFuncSetAttribute(reinterpret_cast<const void *>(&phase2_kernel<ODT, DD>),   \
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);          \
        hipLaunchKernelGGL((phase2_kernel<ODT, DD>), grid, block, lds, stream, p);         \
        return hipGetLastError();
    switch (D) {
        PAV2_P2(64)
        PAV2_P2(80)
        PAV2_P2(96)
        PAV2_P2(112)
        PAV2_P2(120)
        PAV2_P2(128)
        PAV2_P2(192)
        PAV2_P2(256)
    default: return hipErrorInvalidValue;
    }
#undef PAV2_P2
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
