// layer.hip -- per-row roles inside one LSA layer.
//
// Row modes: 0 = not an index owner (an MTP draft that reuses another row's index set, [paper]
// §3.2 "Integration with Multi-Token Prediction"), 1 = flat indexer, 2 = Hierarchical Indexing
// (the sequence is at least hi_min_len long: HI is enabled adaptively beyond its crossover,
// [paper] §3.3 "Design choices", §4.1.2).  Decided on the device from kv_off, so the host never
// reads sequence lengths.
#include "lsa_kernels.hpp"

namespace lsa {

__global__ void row_modes_kernel(RowsDev rows, const int32_t *idx_row, int64_t hi_min_len, int hi_enabled,
                                 uint8_t *row_mode)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows.n_rows)
        return;
    uint8_t mode = 1;
    if (idx_row && idx_row[r] != r) {
        mode = 0;
    } else if (hi_enabled) {
        int32_t b = rows.row_seq[r];
        if (b >= 0 && b < rows.n_seq && rows.kv_off[b + 1] - rows.kv_off[b] >= hi_min_len)
            mode = 2;
    }
    row_mode[r] = mode;
}

hipError_t launch_row_modes(const RowsDev &rows, const int32_t *idx_row, int64_t hi_min_len, int hi_enabled,
                            uint8_t *row_mode, hipStream_t stream)
{
    if (rows.n_rows == 0)
        return hipSuccess;
    hipLaunchKernelGGL(row_modes_kernel, dim3((rows.n_rows + 255) / 256), dim3(256), 0, stream, rows, idx_row,
                       hi_min_len, hi_enabled, row_mode);
    return hipGetLastError();
}

}  // namespace lsa
