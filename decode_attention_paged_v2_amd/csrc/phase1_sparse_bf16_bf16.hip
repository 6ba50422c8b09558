// Block-sparse phase-1 kernel variants for bf16 queries over a bf16
// KV cache (every head size, the dense and compact schedules).  One
// translation unit per dtype pair, so the variants compile in parallel.
#include "phase1_kernel.h"

namespace pav2 {

hipError_t launch_phase1_sparse_bf16_bf16(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream) {
    return launch_d<BF16, BF16, true>(p, head_size, lds_bytes, stream);
}

}  // namespace pav2
