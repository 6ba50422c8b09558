// Debug validator for the device-side data the decode kernels take on trust
// (the pages index the caches with block_tables and seq_lens unchecked, and
// the C ABI does the same): every sequence length lies in
// [0, max_blocks_per_seq * block_size] and every block-table entry a sequence
// uses (column j < ceil(L / block_size)) names a block in [0, num_blocks).
//
// Three small launches on one stream: reset the report, check one sequence
// per wavefront (a 64-bit atomic minimum keeps the first offending
// (sequence, column) whatever the schedule), and expand that key into the
// report.  No memory is allocated.
#include "pav2_internal.h"

namespace pav2 {
namespace {

constexpr unsigned long long kNoKey = ~0ull;

__global__ void check_reset_kernel(long long *report) {
    if (threadIdx.x == 0) {
        report[0] = 0;
        report[1] = (long long)kNoKey;   // the key of the first violation while checking
        report[2] = -1;
        report[3] = 0;
    }
}

__global__ void __launch_bounds__(256) check_kernel(const int32_t *block_tables, const int32_t *seq_lens,
                                                    int num_seqs, int max_blocks_per_seq, int block_size,
                                                    int num_blocks, long long *report) {
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s >= num_seqs) return;
    const int L = seq_lens[s];
    int bad_col = INT32_MAX;   // first offending column; -1: the length itself
    if (L < 0 || (int64_t)L > (int64_t)max_blocks_per_seq * block_size) {
        bad_col = -1;
    } else {
        const int n = (L + block_size - 1) / block_size;
        const int32_t *row = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int j = lane; j < n; j += 64) {
            const int v = row[j];
            if ((v < 0 || v >= num_blocks) && j < bad_col) bad_col = j;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) bad_col = min(bad_col, __shfl_xor(bad_col, off));
    }
    if (bad_col != INT32_MAX && lane == 0) {
        atomicAdd(reinterpret_cast<unsigned long long *>(&report[0]), 1ull);
        const unsigned long long key = ((unsigned long long)s << 32) | (unsigned)(bad_col + 1);
        atomicMin(reinterpret_cast<unsigned long long *>(&report[1]), key);
    }
}

__global__ void check_finish_kernel(const int32_t *block_tables, const int32_t *seq_lens,
                                    int max_blocks_per_seq, long long *report) {
    if (threadIdx.x != 0) return;
    const unsigned long long key = (unsigned long long)report[1];
    if (key == kNoKey) {
        report[1] = -1;
        return;
    }
    const int s = (int)(key >> 32);
    const int col = (int)(key & 0xffffffffu) - 1;
    report[1] = s;
    report[2] = col;
    report[3] = col < 0 ? seq_lens[s] : block_tables[(int64_t)s * max_blocks_per_seq + col];
}

}  // namespace

hipError_t launch_check_inputs(const int32_t *block_tables, const int32_t *seq_lens, int num_seqs,
                               int max_blocks_per_seq, int block_size, int num_blocks, long long *report,
                               hipStream_t stream) {
    hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(64), 0, stream, report);
    if (num_seqs > 0)
        hipLaunchKernelGGL(check_kernel, dim3((num_seqs + 3) / 4), dim3(256), 0, stream, block_tables, seq_lens,
                           num_seqs, max_blocks_per_seq, block_size, num_blocks, report);
    hipLaunchKernelGGL(check_finish_kernel, dim3(1), dim3(64), 0, stream, block_tables, seq_lens,
                       max_blocks_per_seq, report);
    return hipGetLastError();
}

}  // namespace pav2
