// Phase-1 kernel variants for f16 queries over a f16 KV cache (every
// head size, schedule and block-size specialisation of that pair).  One
// translation unit per dtype pair, so the variants compile in parallel.
#include "phase1_kernel.h"

namespace pav2 {

hipError_t launch_phase1_f16_f16(const Phase1Params &p, int head_size, int lds_bytes, hipStream_t stream) {
    return launch_d<F16, F16, false>(p, head_size, lds_bytes, stream);
}

}  // namespace pav2
