// lsa_kernels.hpp -- host-side launchers of the liblsa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lsa_dev.hpp"

namespace lsa {

// Row gating for the layer: when row_mode != nullptr, only rows with row_mode[r] == want run.
struct RowGate {
    const uint8_t *row_mode;
    int want;
};

// --- top-k (topk.hip)
// Columns of a row are cut into chunks of chunk_elems; each chunk has its own histogram slot.
struct TopkGeom {
    int64_t chunk_elems;
    int n_chunks;
};
struct TopkState;
struct TopkWs {
    TopkState *state;   // [n_rows] search state
    uint32_t *hist;     // [n_rows][n_chunks][2048] suffix histograms of the current pass
    uint32_t *chunk_gt; // [n_rows][n_chunks] keys known to be picked
    uint32_t *chunk_eq; // [n_rows][n_chunks] keys equal to the threshold (when ties are split)
};
TopkGeom topk_geometry(int n_rows, int64_t n_cols);
TopkWs topk_carve(void *ws, int n_rows, int n_chunks);
size_t topk_workspace_bytes_geo(int n_rows, int n_chunks);
size_t topk_workspace_bytes(int n_rows, int64_t n_cols, int k);
// k <= 4096: two-level selection (segments selected in registers, no per-chunk histograms; a
// caller-chosen chunking and pre-computed pass-0 histograms are not used).
bool topk_two_level(int k);
hipError_t launch_topk(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M,
                       int P, int k, int32_t *idx, void *ws, RowGate gate, hipStream_t stream);
// Same, over a caller-chosen chunking; pass0_done: the pass-0 suffix histograms are already in ws.
hipError_t launch_topk_geo(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M,
                           int P, int k, int32_t *idx, void *ws, TopkGeom geo, bool pass0_done, RowGate gate,
                           hipStream_t stream);
constexpr int kTopkBins = 2048;

// lh[] (kTopkBins LDS counters) -> out[b] = sum of lh[b'] for b' >= b (the keys in bin b or above).
// Every thread of a block of `nthreads` (a multiple of 64 dividing kTopkBins) calls it; `part` is
// LDS scratch of nthreads words.  PACKED: lh holds two 16-bit counters per word (bin b in half
// b % 2 of word b / 2).
template <bool PACKED = false>
__device__ inline uint32_t hist_bin(const uint32_t *lh, int b)
{
    if constexpr (PACKED)
        return (lh[b >> 1] >> (16 * (b & 1))) & 0xffffu;
    else
        return lh[b];
}

template <bool PACKED = false>
__device__ inline void store_suffix_hist(const uint32_t *lh, uint32_t *part, uint32_t *__restrict__ out,
                                         int nthreads)
{
    const int t = threadIdx.x;
    const int per = kTopkBins / nthreads;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i)
        s += hist_bin<PACKED>(lh, t * per + i);
    part[t] = s;
    __syncthreads();
    if (t < kWave) {
        // Exclusive suffix sums of the parts (part t covers bins [t*per, (t+1)*per)), from the top,
        // one group of 64 parts at a time (lane 0 takes the highest part of the group).
        uint32_t run = 0;
        for (int base = nthreads - kWave; base >= 0; base -= kWave) {
            const int idx = base + (kWave - 1 - t);
            const uint32_t v = part[idx];
            uint32_t incl = v;
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t y = (uint32_t)__shfl_up((int)incl, o, kWave);
                if (t >= o)
                    incl += y;
            }
            part[idx] = run + incl - v;
            run += (uint32_t)__shfl((int)incl, kWave - 1, kWave);
        }
    }
    __syncthreads();
    uint32_t acc = part[t];
    for (int i = per - 1; i >= 0; --i) {
        acc += hist_bin<PACKED>(lh, t * per + i);
        out[t * per + i] = acc;
    }
}

// --- indexer scoring (index_score.hip)
enum ScoreMode { kScoreFlat = 0, kScorePaged = 1 };

hipError_t launch_index_score(int dtype, const RowsDev &rows, int64_t max_kv_len, const void *q_idx, const float *w,
                              const void *k_idx, int n_heads, int head_dim, int k_sink, int k_swa,
                              const int32_t *pages, int M, int P, float *scores, int64_t ld, RowGate gate,
                              hipStream_t stream, uint32_t *topk_hist = nullptr);
// Chunking of the scoring grid (one chunk per block of a row); the fused top-K histograms use it.
TopkGeom score_geometry(int dtype, int n_rows, int64_t n_cols);
bool index_score_supported(int dtype, int n_heads, int head_dim);

// HI stage 1: page scores (sums of sub-block scores per page), -inf for non-causal pages.
hipError_t launch_page_scores(int dtype, const RowsDev &rows, int64_t max_kv_len, const int64_t *sb_off,
                              const void *q_idx, const float *w, const void *k_mean, int n_heads, int head_dim,
                              int P, int B, float *page_scores, int64_t ld_ps, RowGate gate, hipStream_t stream);

// --- sub-block means (hi.hip)
hipError_t launch_page_means(int dtype, int n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                             int head_dim, int B, int64_t max_kv_len, int64_t first_token, void *k_mean,
                             hipStream_t stream);

// --- attention (attn.hip)
size_t attn_workspace_bytes(int dtype, int n_rows, int n_heads, int d_v, int k_total);
bool attn_supported(int dtype, int n_heads, int d_qk, int d_v, int k_sparse, int k_total);
hipError_t launch_hybrid_attn(int dtype, const RowsDev &rows, const void *q, const void *kv, int n_heads, int d_qk,
                              int d_v, float scale, int k_sink, int k_swa, int k_sparse, const int32_t *idx,
                              const int32_t *idx_row, void *out, float *lse, void *ws, hipStream_t stream);

// --- layer helpers (layer.hip)
hipError_t launch_row_modes(const RowsDev &rows, const int32_t *idx_row, int64_t hi_min_len, int hi_enabled,
                            uint8_t *row_mode, hipStream_t stream);

// Rounds a byte count up to the workspace alignment.
inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace lsa
