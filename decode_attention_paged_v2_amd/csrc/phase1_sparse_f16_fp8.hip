// Block-sparse phase-1 kernel variants for f16 queries over a fp8 e4m3
// KV cache (every head size, the dense and compact schedules).  One
// translation unit per dtype pair, so the variants compile in parallel.
#include "phase1_kernel.h"

namespace pav2 {

hipError_t launch_phase1_sparse_f16_fp8(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream) {
    return launch_d<F16, FP8, true>(p, head_size, lds_bytes, stream);
}

}  // namespace pav2
