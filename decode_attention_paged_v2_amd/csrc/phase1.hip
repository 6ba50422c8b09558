// Phase 1 of PagedAttention V2 decode: dispatch of a launch onto the kernel
// variants of its (query dtype, kv cache dtype) pair.  The kernel itself is
// in phase1_kernel.h; each pair's variants are built in their own
// translation unit (phase1_<query>_<cache>.hip, and the block-sparse ones in
// phase1_sparse_<query>_<cache>.hip).
#include "pav2_internal.h"

namespace pav2 {

hipError_t launch_phase1_f32_f32(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_f16_f16(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_bf16_bf16(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_f32_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_f16_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_bf16_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_sparse_f32_f32(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_sparse_f16_f16(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_sparse_bf16_bf16(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_sparse_f32_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_sparse_f16_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);
hipError_t launch_phase1_sparse_bf16_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream);

hipError_t launch_phase1(const Phase1Params &p, int qdt, int kvdt, int head_size, int waves,
                         int lds_bytes, hipStream_t stream) {
    if (waves != kPhase1Waves) return hipErrorInvalidValue;
    if (p.sp_vert_stride > 1) {   // block-sparse pattern
        if (qdt == F32 && kvdt == F32) return launch_phase1_sparse_f32_f32(p, head_size, lds_bytes, stream);
        if (qdt == F16 && kvdt == F16) return launch_phase1_sparse_f16_f16(p, head_size, lds_bytes, stream);
        if (qdt == BF16 && kvdt == BF16) return launch_phase1_sparse_bf16_bf16(p, head_size, lds_bytes, stream);
        if (qdt == F32 && kvdt == FP8) return launch_phase1_sparse_f32_fp8(p, head_size, lds_bytes, stream);
        if (qdt == F16 && kvdt == FP8) return launch_phase1_sparse_f16_fp8(p, head_size, lds_bytes, stream);
        if (qdt == BF16 && kvdt == FP8) return launch_phase1_sparse_bf16_fp8(p, head_size, lds_bytes, stream);
        return hipErrorInvalidValue;
    }
    if (qdt == F32 && kvdt == F32) return launch_phase1_f32_f32(p, head_size, lds_bytes, stream);
    if (qdt == F16 && kvdt == F16) return launch_phase1_f16_f16(p, head_size, lds_bytes, stream);
    if (qdt == BF16 && kvdt == BF16) return launch_phase1_bf16_bf16(p, head_size, lds_bytes, stream);
    if (qdt == F32 && kvdt == FP8) return launch_phase1_f32_fp8(p, head_size, lds_bytes, stream);
    if (qdt == F16 && kvdt == FP8) return launch_phase1_f16_fp8(p, head_size, lds_bytes, stream);
    if (qdt == BF16 && kvdt == FP8) return launch_phase1_bf16_fp8(p, head_size, lds_bytes, stream);
    return hipErrorInvalidValue;
}

}  // namespace pav2
