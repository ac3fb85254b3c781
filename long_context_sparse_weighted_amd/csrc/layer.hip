// layer.hip -- per-row roles inside one LSA layer.
//
// Row modes: 0 = not an index owner (an MTP draft that reuses another row's index set, [paper]
// §3.2 "Integration with Multi-Token Prediction"), 1 = flat indexer, 2 = Hierarchical Indexing
// (the sequence is at least hi_min_len long: HI is enabled adaptively beyond its crossover,
// [paper] §3.3 "Design choices", §4.1.2).  Decided on the device from kv_off, so the host never
// reads sequence lengths.
#include "lsa_kernels.hpp"
#include "topk_block.hpp"

namespace lsa {

// One block of 1024 threads: thread t decides the modes of rows [t per, t per + per) and the block scan
// of the per-thread counts places the flat and HI rows in their lists in ascending row order.
constexpr int kModeThreads = 1024;

__global__ __launch_bounds__(kModeThreads) void row_modes_kernel(RowsDev rows, const int32_t *idx_row,
                                                                 int64_t hi_min_len, int hi_enabled,
                                                                 uint8_t *row_mode, int32_t *lists, int32_t *counts,
                                                                 int k_sink, int k_swa, int64_t fused_cols,
                                                                 int32_t *table, int64_t table_cap)
{
    __shared__ uint32_t scan[2 * kModeThreads / kWave];
    const int n = rows.n_rows;
    const int per = (n + kModeThreads - 1) / kModeThreads;
    const int r0 = threadIdx.x * per;
    auto mode_of = [&](int r) -> uint8_t {
        if (idx_row && idx_row[r] != r)
            return 0;
        if (hi_enabled) {
            const int32_t b = rows.row_seq[r];
            if (b >= 0 && b < rows.n_seq && rows.kv_off[b + 1] - rows.kv_off[b] >= hi_min_len)
                return 2;
        }
        return 1;
    };
    uint32_t c1 = 0, c2 = 0;
    for (int i = 0; i < per; ++i) {
        const int r = r0 + i;
        if (r < n) {
            const uint8_t m = mode_of(r);
            row_mode[r] = m;
            c1 += m == 1 ? 1u : 0u;
            c2 += m == 2 ? 1u : 0u;
        }
    }
    uint32_t e1, e2, t1, t2;
    block_scan2<kModeThreads>(c1, c2, e1, e2, t1, t2, scan);
    for (int i = 0; i < per; ++i) {
        const int r = r0 + i;
        if (r < n) {
            const uint8_t m = row_mode[r];  // (this thread's own write)
            if (m == 1)
                lists[e1++] = r;
            else if (m == 2)
                lists[n + e2++] = r;
        }
    }
    if (threadIdx.x == 0)
        counts[0] = (int32_t)t1, counts[1] = (int32_t)t2;
    if (fused_cols <= 0)
        return;
    // The fused pass's blocks with work: fused_row_lists(r) chunks of each flat row, in row order.
    uint32_t nb = 0;
    for (int i = 0; i < per; ++i) {
        const int r = r0 + i;
        if (r < n && row_mode[r] == 1)
            nb += (uint32_t)fused_row_lists(rows, r, k_sink, k_swa, fused_cols);
    }
    uint32_t eb, e0, tb, t0;
    __syncthreads();  // (scan scratch reuse)
    block_scan2<kModeThreads>(nb, 0u, eb, e0, tb, t0, scan);
    for (int i = 0; i < per; ++i) {
        const int r = r0 + i;
        if (r < n && row_mode[r] == 1) {
            const int64_t nl = fused_row_lists(rows, r, k_sink, k_swa, fused_cols);
            for (int64_t c = 0; c < nl; ++c, ++eb)
                if ((int64_t)eb < table_cap)
                    table[2 * (int64_t)eb] = r, table[2 * (int64_t)eb + 1] = (int32_t)c;
        }
    }
    if (threadIdx.x == 0)
        counts[2] = (int32_t)((int64_t)tb < table_cap ? (int64_t)tb : table_cap);
}

hipError_t launch_row_modes(const RowsDev &rows, const int32_t *idx_row, int64_t hi_min_len, int hi_enabled,
                            uint8_t *row_mode, int32_t *lists, int32_t *counts, int k_sink, int k_swa,
                            int64_t fused_cols, int32_t *table, int64_t table_cap, hipStream_t stream)
{
    if (rows.n_rows == 0)
        return hipSuccess;
    hipLaunchKernelGGL(row_modes_kernel, dim3(1), dim3(kModeThreads), 0, stream, rows, idx_row, hi_min_len,
                       hi_enabled, row_mode, lists, counts, k_sink, k_swa, fused_cols, table, table_cap);
    return hipGetLastError();
}

}  // namespace lsa
