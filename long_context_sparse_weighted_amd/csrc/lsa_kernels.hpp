// lsa_kernels.hpp -- host-side launchers of the liblsa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lsa.h"
#include "lsa_dev.hpp"

namespace lsa {

// Row gating for the layer: when row_mode != nullptr, only rows with row_mode[r] == want run.
// list / count (optional, streaming scoring kernels only): the rows with row_mode[r] == want in ascending
// order and their number, so that the blocks of those rows can be launched first.
// table / table_count (optional, the fused flat pass only): its blocks that have work, as (row, chunk)
// pairs in order, so that those come first and no block without work is launched among them.
struct RowGate {
    const uint8_t *row_mode;
    int want;
    const int32_t *list = nullptr;
    const int32_t *count = nullptr;
    const int32_t *table = nullptr;
    const int32_t *table_count = nullptr;
};

// Per-row input sizes of the candidate-list levels after a fused first level (on = false: every row has
// the uniform count): row r starts with fused_row_lists(rows, r, k_sink, k_swa, cols) lists of k.
struct ListCount {
    RowsDev rows;
    int k_sink, k_swa;
    int64_t cols;
    bool on;
};

// --- top-k (topk.hip): exact selection of the k best (score desc, position asc), 1 <= k <= 4096.
// First-level candidate lists computed elsewhere (n_seg lists of k per row): their workspace, the
// buffers to fill, and the remaining levels down to idx.
size_t topk_lists_workspace_bytes(int n_rows, int64_t n_seg, int k);
void topk_first_lists(void *ws, int n_rows, int64_t n_seg, int k, uint32_t **key, int32_t **pos, int64_t *ld);
hipError_t launch_topk_lists(int n_rows, int64_t n_seg, int k, void *ws, int32_t *idx, RowGate gate, ListCount cnt,
                             hipStream_t stream);
size_t topk_workspace_bytes(int n_rows, int64_t n_cols, int k);
hipError_t launch_topk(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M,
                       int P, int k, int32_t *idx, void *ws, RowGate gate, hipStream_t stream);

// --- indexer scoring (index_score.hip)
enum ScoreMode { kScoreFlat = 0, kScorePaged = 1 };

hipError_t launch_index_score(int dtype, const RowsDev &rows, int64_t max_kv_len, const void *q_idx, const float *w,
                              const void *k_idx, int n_heads, int head_dim, int k_sink, int k_swa,
                              const int32_t *pages, int M, int P, float *scores, int64_t ld, RowGate gate,
                              hipStream_t stream);
bool index_score_supported(int dtype, int n_heads, int head_dim);

// HI stage 1: page scores (sums of sub-block scores per page), -inf for non-causal pages.
hipError_t launch_page_scores(int dtype, const RowsDev &rows, int64_t max_kv_len, const int64_t *sb_off,
                              const void *q_idx, const float *w, const void *k_mean, int n_heads, int head_dim,
                              int P, int B, float *page_scores, int64_t ld_ps, RowGate gate, hipStream_t stream);

// --- fused flat scoring + first top-K level (index_score.hip), for rows scored one by one (fewer than
// 64 rows: no 16-row groups); segments of index_select_fused_cols() columns
bool index_select_fusable(int dtype, int n_rows, int n_seq, int n_heads, int head_dim, int k);
int64_t index_select_fused_segments(int64_t n_cols);
int64_t index_select_fused_cols(int64_t n_rows, int64_t n_cols);      // bf16 chunk width: 8192 or 16384
int64_t index_select_fused_cols_fp8(int64_t n_rows, int64_t n_cols);  // FP8 chunk width: 8192 or 16384
hipError_t launch_index_select_fused(const RowsDev &rows, const void *q_idx, const float *w, const void *k_idx,
                                     int k_sink, int k_swa, int64_t n_cols, int64_t cols, int k, uint32_t *sel_key,
                                     int32_t *sel_pos, int64_t sel_ld, RowGate gate, hipStream_t stream);

// --- FP8 indexer (index_score.hip): E4M3 codes, one power-of-two scale per vector
hipError_t launch_index_score_fp8(const RowsDev &rows, const uint8_t *q8, const float *q_scale, const float *w,
                                  const uint8_t *k8, const float *k_scale, int k_sink, int k_swa,
                                  const int32_t *pages, int M, int P, float *scores, int64_t ld, hipStream_t stream);
hipError_t launch_quantize_fp8(int dtype, int64_t n_vec, int dim, const void *x, uint8_t *codes, float *scale,
                               hipStream_t stream);
// FP8 scoring fused with the first top-K level (flat columns; segments as for the bf16 fused pass)
hipError_t launch_index_select_fused_fp8(const RowsDev &rows, const uint8_t *q8, const float *q_scale, const float *w,
                                         const uint8_t *k8, const float *k_scale, int k_sink, int k_swa,
                                         int64_t n_cols, int64_t cols, int k, uint32_t *sel_key, int32_t *sel_pos,
                                         int64_t sel_ld, hipStream_t stream);

// --- sub-block means (hi.hip)
hipError_t launch_page_means(int dtype, int n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                             int head_dim, int B, int64_t max_kv_len, int64_t first_token, int64_t n_new,
                             void *k_mean, hipStream_t stream);

// --- attention (attn.hip)
size_t attn_workspace_bytes(int dtype, int n_rows, int n_heads, int d_v, int k_total);
bool attn_supported(int dtype, int n_heads, int d_qk, int d_v, int k_sparse, int k_total);
hipError_t launch_hybrid_attn(int dtype, const RowsDev &rows, const void *q, const void *kv, int n_heads, int d_qk,
                              int d_v, float scale, int k_sink, int k_swa, int k_sparse, const int32_t *idx,
                              const int32_t *idx_row, void *out, float *lse, void *ws, hipStream_t stream);

// --- layer helpers (layer.hip)
// Also writes, for modes 1 and 2, the rows of that mode in ascending order (lists [2][n_rows]) and their
// numbers (counts[0..1]); with fused_cols > 0 also the (row, chunk) pairs of the fused flat pass's blocks
// that have work (table [2 * table_cap], fused_row_lists of each flat row, rows ascending) and their
// number (counts[2]; at most table_cap).
hipError_t launch_row_modes(const RowsDev &rows, const int32_t *idx_row, int64_t hi_min_len, int hi_enabled,
                            uint8_t *row_mode, int32_t *lists, int32_t *counts, int k_sink, int k_swa,
                            int64_t fused_cols, int32_t *table, int64_t table_cap, hipStream_t stream);

// Rounds a byte count up to the workspace alignment.
inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Records msg as the calling thread's lsa_last_error() text and returns code.
int set_error(int code, const char *msg);

// The host-side checks of lsa_index_topk (errors recorded as lsa_last_error() text); on LSA_OK,
// *ws_bytes is the workspace its launch needs.  Touches no HIP call.
int index_topk_check(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                     int n_heads, int head_dim, lsa_budget_t budget, const int32_t *idx, size_t *ws_bytes);

}  // namespace lsa
