// Measurement aid, not part of the attention path: a read-only sweep of
// device memory with 16-byte vector loads, for the achievable read bandwidth
// of the chip (non-temporal loads, as phase 1 streams K/V) and for flushing
// the caches between timed steps (ordinary loads allocate in L2 and the
// Infinity Cache and so evict what they held, without leaving dirty lines).
#include "pav2_internal.h"

namespace pav2 {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per lane

template <bool NT>
__global__ void __launch_bounds__(kStreamThreads) read_stream_kernel(const u32x4 *src, int64_t n16, uint32_t *sink) {
    // each workgroup sweeps one contiguous slab, kStreamUnroll loads per lane at a time
    const int64_t per_wg = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = per_wg * blockIdx.x;
    const int64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
    uint32_t acc = 0;
    for (int64_t base = lo + threadIdx.x; base < hi; base += (int64_t)kStreamThreads * kStreamUnroll) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int k = 0; k < kStreamUnroll; ++k) {
            const int64_t i = base + (int64_t)k * kStreamThreads;
            v[k] = u32x4{0u, 0u, 0u, 0u};
            if (i < hi) v[k] = NT ? __builtin_nontemporal_load(src + i) : src[i];
        }
#pragma unroll
        for (int k = 0; k < kStreamUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    // keeps the loads live; a store only for one data-dependent value
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_stream(const void *src, int64_t bytes, bool nontemporal, uint32_t *sink, int workgroups,
                              hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const u32x4 *p = static_cast<const u32x4 *>(src);
    if (nontemporal)
        hipLaunchKernelGGL(read_stream_kernel<true>, dim3(workgroups), dim3(kStreamThreads), 0, stream, p, n16, sink);
    else
        hipLaunchKernelGGL(read_stream_kernel<false>, dim3(workgroups), dim3(kStreamThreads), 0, stream, p, n16, sink);
    return hipGetLastError();
}

}  // namespace pav2
