// api.cpp -- the extern "C" boundary of liblsa (declared in include/lsa.h).
//
// Every entry point checks its scalars and host structs first and returns LSA_ERR_INVALID /
// LSA_ERR_UNSUPPORTED / LSA_ERR_WORKSPACE before touching the HIP runtime; only then are kernels
// enqueued on the caller's stream.  The library allocates nothing: scratch is carved from the
// caller's workspace.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/lsa.h"
#include "lsa_kernels.hpp"

using namespace lsa;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = 0;
    return LSA_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(LSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr int64_t kMaxGridRows = 65535;

int check_rows(const lsa_rows_t *rows)
{
    if (!rows)
        return fail(LSA_ERR_INVALID, "rows is NULL");
    if (rows->n_seq < 0 || rows->n_rows < 0 || rows->max_kv_len < 0)
        return fail(LSA_ERR_INVALID, "negative n_seq / n_rows / max_kv_len");
    if (rows->n_rows > 0 && (!rows->kv_off || !rows->row_seq || !rows->row_pos))
        return fail(LSA_ERR_INVALID, "rows: kv_off / row_seq / row_pos must be device pointers");
    if (rows->n_rows > kMaxGridRows)
        return fail(LSA_ERR_UNSUPPORTED, "n_rows %d exceeds %lld", rows->n_rows, (long long)kMaxGridRows);
    if (rows->min_kv_len < 0 || rows->min_kv_len > rows->max_kv_len)
        return fail(LSA_ERR_INVALID, "min_kv_len must lie in [0, max_kv_len]");
    if (rows->max_kv_len >= (int64_t)1 << 31)
        return fail(LSA_ERR_UNSUPPORTED, "max_kv_len must be below 2^31");
    return LSA_OK;
}

int check_budget(lsa_budget_t b)
{
    if (b.k_sink < 0 || b.k_swa < 0 || b.k_sparse < 0)
        return fail(LSA_ERR_INVALID, "budget entries must be >= 0");
    return LSA_OK;
}

RowsDev to_dev(const lsa_rows_t *rows)
{
    RowsDev d;
    d.kv_off = rows->kv_off;
    d.row_seq = rows->row_seq;
    d.row_pos = rows->row_pos;
    d.n_rows = rows->n_rows;
    d.n_seq = rows->n_seq;
    return d;
}

bool aligned256(const void *p) { return ((uintptr_t)p & 255) == 0; }

// Sequential carving of the caller's workspace.
struct Carver {
    char *p;
    size_t used = 0;
    explicit Carver(void *base) : p((char *)base) {}
    void *take(size_t bytes)
    {
        void *r = p ? p + used : nullptr;
        used += align_up(bytes);
        return r;
    }
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int check_page_geometry(int dtype, int32_t P, int32_t B, int32_t M)
{
    if (P <= 0 || B <= 0 || M <= 0)
        return fail(LSA_ERR_INVALID, "P, B and M must be positive");
    if (P % B != 0)
        return fail(LSA_ERR_INVALID, "B (%d) must divide P (%d)", B, P);
    if (P % 16 != 0)
        return fail(LSA_ERR_UNSUPPORTED, "P must be a multiple of 16");
    if ((int64_t)M * P >= ((int64_t)1 << 31))
        return fail(LSA_ERR_INVALID, "M*P overflows int32");
    if (dtype == LSA_BF16 && !(is_pow2(P / B) && P / B <= 16))
        return fail(LSA_ERR_UNSUPPORTED, "bf16 page scoring needs P/B a power of two <= 16");
    if (M > 4096)
        return fail(LSA_ERR_UNSUPPORTED, "M above 4096");
    return LSA_OK;
}

// Workspace layout of lsa_layer_fwd.
struct LayerWs {
    uint8_t *row_mode;
    int32_t *row_lists;   // [2][n_rows]: flat rows, HI rows (ascending)
    int32_t *row_counts;  // [3]: flat rows, HI rows, fused-pass blocks with work
    int32_t *fused_table; // [2 * fused_cap]: (row, chunk) of those blocks
    int64_t fused_cap;
    int64_t fused_cols;   // chunk width of the fused flat pass (0: not fused)
    void *topk_ws;
    float *page_scores;
    int32_t *pages;
    void *page_topk_ws;
    float *comp_scores;
    void *attn_ws;
    size_t bytes;
};

// The fused flat pass works on fixed chunks of columns per block (8192, or 16384 for long rows): it needs
// rows that are scored one by one, and enough chunks to give every CU at least one block (a 32-row batch
// from 64K columns on; below that the separate passes, whose chunks shrink with the work, are faster).
bool flat_fused(int dtype, const lsa_rows_t *rows, int n_heads, int head_dim, int k)
{
    return index_select_fusable(dtype, rows->n_rows, rows->n_seq, n_heads, head_dim, k) &&
           (int64_t)rows->n_rows * index_select_fused_segments(rows->max_kv_len) >= 256;
}
bool flat_fused(const lsa_layer_cfg_t *cfg, const lsa_rows_t *rows)
{
    return flat_fused(cfg->dtype, rows, cfg->n_heads_idx, cfg->head_dim_idx, cfg->budget.k_sparse);
}

// Chunks of the fused pass over ld columns.
int64_t flat_fused_segments(const lsa_rows_t *rows, int64_t ld, int64_t *cols)
{
    *cols = index_select_fused_cols(rows->n_rows, ld);
    return (ld + *cols - 1) / *cols;
}

// The same for the FP8 fused pass, whose 16384-column form needs two blocks per CU.
int64_t fp8_fused_segments(const lsa_rows_t *rows, int64_t ld, int64_t *cols)
{
    *cols = index_select_fused_cols_fp8(rows->n_rows, ld);
    return (ld + *cols - 1) / *cols;
}

// Workspace of the flat selection (lsa_index_topk and the layer's flat rows): candidate lists of the
// fused pass, or the scores and the top-K lists of the separate passes; the scores come first.
size_t flat_select_bytes(int dtype, const lsa_rows_t *rows, int n_heads, int head_dim, int k, size_t *scores_bytes)
{
    const int64_t ld = rows->max_kv_len > 0 ? rows->max_kv_len : 1;
    if (flat_fused(dtype, rows, n_heads, head_dim, k)) {
        *scores_bytes = 0;
        int64_t cols;
        return topk_lists_workspace_bytes(rows->n_rows, flat_fused_segments(rows, ld, &cols), k);
    }
    *scores_bytes = align_up(sizeof(float) * (size_t)rows->n_rows * (size_t)ld);
    return *scores_bytes + topk_workspace_bytes(rows->n_rows, ld, k);
}

hipError_t launch_flat_select(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                              int n_heads, int head_dim, lsa_budget_t bud, int32_t *idx, void *ws, RowGate gate,
                              hipStream_t stream)
{
    const RowsDev rd = to_dev(rows);
    const int64_t ld = rows->max_kv_len > 0 ? rows->max_kv_len : 1;
    if (flat_fused(dtype, rows, n_heads, head_dim, bud.k_sparse)) {
        // scoring and the first top-K level in one pass; the scores never leave the chip
        int64_t cols;
        const int64_t n_seg = flat_fused_segments(rows, ld, &cols);
        uint32_t *sk;
        int32_t *sp;
        int64_t sld;
        topk_first_lists(ws, rows->n_rows, n_seg, bud.k_sparse, &sk, &sp, &sld);
        hipError_t e = launch_index_select_fused(rd, q_idx, w, k_idx, bud.k_sink, bud.k_swa, ld, cols, bud.k_sparse,
                                                 sk, sp, sld, gate, stream);
        if (e != hipSuccess)
            return e;
        return launch_topk_lists(rows->n_rows, n_seg, bud.k_sparse, ws, idx, gate,
                                 ListCount{rd, bud.k_sink, bud.k_swa, cols, true}, stream);
    }
    size_t sb;
    (void)flat_select_bytes(dtype, rows, n_heads, head_dim, bud.k_sparse, &sb);
    float *scores = (float *)ws;
    hipError_t e = launch_index_score(dtype, rd, rows->max_kv_len, q_idx, w, k_idx, n_heads, head_dim, bud.k_sink,
                                      bud.k_swa, nullptr, 0, 1, scores, ld, gate, stream);
    if (e != hipSuccess)
        return e;
    return launch_topk(rows->n_rows, scores, ld, ld, nullptr, 0, 1, bud.k_sparse, idx, (char *)ws + sb, gate, stream);
}

LayerWs layer_ws_layout(const lsa_layer_cfg_t *cfg, const lsa_rows_t *rows, bool use_hi, void *base)
{
    Carver c(base);
    LayerWs w{};
    const int64_t n = rows->n_rows;
    const int k_total = cfg->budget.k_sink + cfg->budget.k_swa + cfg->budget.k_sparse;
    if (cfg->is_owner) {
        w.row_mode = (uint8_t *)c.take((size_t)n);
        w.row_lists = (int32_t *)c.take(sizeof(int32_t) * 2 * (size_t)n);
        w.row_counts = (int32_t *)c.take(sizeof(int32_t) * 4);
        w.fused_cols = 0;
        w.fused_cap = 0;
        if (flat_fused(cfg, rows)) {
            const int64_t segs = flat_fused_segments(rows, rows->max_kv_len > 0 ? rows->max_kv_len : 1, &w.fused_cols);
            w.fused_cap = segs * n;
        }
        w.fused_table = (int32_t *)c.take(sizeof(int32_t) * 2 * (size_t)w.fused_cap);
        // The flat and the HI token top-K share one workspace.  Rows scored one by one take the fused
        // scoring + first top-K level, which writes candidate lists instead of scores.
        size_t sb;
        size_t tk = flat_select_bytes(cfg->dtype, rows, cfg->n_heads_idx, cfg->head_dim_idx, cfg->budget.k_sparse, &sb);
        if (use_hi) {
            const size_t hk = topk_workspace_bytes((int)n, (int64_t)cfg->M * cfg->P, cfg->budget.k_sparse);
            tk = hk > tk ? hk : tk;
        }
        w.topk_ws = c.take(tk);
        if (use_hi) {
            int64_t n_pages = ceil_div(rows->max_kv_len, cfg->P);
            w.page_scores = (float *)c.take(sizeof(float) * (size_t)n * (size_t)n_pages);
            w.pages = (int32_t *)c.take(sizeof(int32_t) * (size_t)n * (size_t)cfg->M);
            w.page_topk_ws = c.take(topk_workspace_bytes((int)n, n_pages, cfg->M));
            w.comp_scores = (float *)c.take(sizeof(float) * (size_t)n * (size_t)cfg->M * (size_t)cfg->P);
        }
    }
    w.attn_ws = c.take(attn_workspace_bytes(cfg->dtype, (int)n, cfg->n_heads, cfg->d_v, k_total));
    w.bytes = c.used;
    return w;
}

int check_layer_cfg(const lsa_layer_cfg_t *cfg)
{
    if (!cfg)
        return fail(LSA_ERR_INVALID, "cfg is NULL");
    if (cfg->dtype != LSA_F32 && cfg->dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (int st = check_budget(cfg->budget))
        return st;
    if (cfg->n_heads <= 0 || cfg->d_qk <= 0 || cfg->d_v <= 0)
        return fail(LSA_ERR_INVALID, "attention shape must be positive");
    const int k_total = cfg->budget.k_sink + cfg->budget.k_swa + cfg->budget.k_sparse;
    if (!attn_supported(cfg->dtype, cfg->n_heads, cfg->d_qk, cfg->d_v, cfg->budget.k_sparse, k_total))
        return fail(LSA_ERR_UNSUPPORTED, "attention shape (H=%d, d_qk=%d, d_v=%d) not compiled for this dtype",
                    cfg->n_heads, cfg->d_qk, cfg->d_v);
    if (cfg->is_owner) {
        if (cfg->budget.k_sparse < 1 || cfg->budget.k_sparse > 4096)
            return fail(LSA_ERR_UNSUPPORTED, "k_sparse must be in [1, 4096]");
        if (!index_score_supported(cfg->dtype, cfg->n_heads_idx, cfg->head_dim_idx))
            return fail(LSA_ERR_UNSUPPORTED, "indexer shape (%d heads, dim %d) not compiled for this dtype",
                        cfg->n_heads_idx, cfg->head_dim_idx);
    }
    return LSA_OK;
}

int check_index_topk(int dtype, const lsa_rows_t *rows, int32_t n_heads, int32_t head_dim, int32_t k)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (int st = check_rows(rows))
        return st;
    if (!index_score_supported(dtype, n_heads, head_dim))
        return fail(LSA_ERR_UNSUPPORTED, "indexer shape (%d heads, dim %d) not compiled for this dtype", n_heads,
                    head_dim);
    if (k < 1 || k > 4096)
        return fail(LSA_ERR_UNSUPPORTED, "k_sparse must be in [1, 4096]");
    return LSA_OK;
}

}  // namespace

namespace lsa {

int set_error(int code, const char *msg) { return fail(code, "%s", msg); }

int index_topk_check(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                     int n_heads, int head_dim, lsa_budget_t budget, const int32_t *idx, size_t *ws_bytes)
{
    if (int st = check_index_topk(dtype, rows, n_heads, head_dim, budget.k_sparse))
        return st;
    if (int st = check_budget(budget))
        return st;
    if (rows->n_rows > 0 && (!q_idx || !w || !k_idx || !idx))
        return fail(LSA_ERR_INVALID, "q_idx, w, k_idx and idx must be device pointers");
    size_t sb;
    *ws_bytes = flat_select_bytes(dtype, rows, n_heads, head_dim, budget.k_sparse, &sb);
    return LSA_OK;
}

}  // namespace lsa

extern "C" {

const char *lsa_status_string(int status)
{
    switch (status) {
    case LSA_OK:
        return "ok";
    case LSA_ERR_INVALID:
        return "invalid argument";
    case LSA_ERR_UNSUPPORTED:
        return "unsupported shape or dtype";
    case LSA_ERR_WORKSPACE:
        return "workspace too small";
    case LSA_ERR_HIP:
        return "HIP runtime error";
    default:
        return "unknown status";
    }
}

const char *lsa_last_error(void) { return g_err; }

int lsa_index_score(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                    int32_t n_heads, int32_t head_dim, lsa_budget_t budget, const int32_t *pages, int32_t M,
                    int32_t P, float *scores, int64_t ld_scores, hipStream_t stream)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (int st = check_rows(rows))
        return st;
    if (int st = check_budget(budget))
        return st;
    if (!index_score_supported(dtype, n_heads, head_dim))
        return fail(LSA_ERR_UNSUPPORTED, "indexer shape (%d heads, dim %d) not compiled for this dtype", n_heads,
                    head_dim);
    if (rows->n_rows > 0 && (!q_idx || !w || !k_idx || !scores))
        return fail(LSA_ERR_INVALID, "q_idx, w, k_idx and scores must be device pointers");
    if (pages) {
        if (M <= 0 || P <= 0)
            return fail(LSA_ERR_INVALID, "page mode needs M > 0 and P > 0");
        if (P % 16 != 0)
            return fail(LSA_ERR_UNSUPPORTED, "page mode needs P %% 16 == 0");
        if ((int64_t)M * P >= ((int64_t)1 << 31))
            return fail(LSA_ERR_INVALID, "M*P overflows int32");
        if (ld_scores < (int64_t)M * P)
            return fail(LSA_ERR_INVALID, "ld_scores %lld < M*P", (long long)ld_scores);
    } else if (ld_scores < rows->max_kv_len) {
        return fail(LSA_ERR_INVALID, "ld_scores %lld < max_kv_len %lld", (long long)ld_scores,
                    (long long)rows->max_kv_len);
    }
    if (ld_scores >= ((int64_t)1 << 31))
        return fail(LSA_ERR_UNSUPPORTED, "ld_scores must be below 2^31");
    hipError_t e = launch_index_score(dtype, to_dev(rows), rows->max_kv_len, q_idx, w, k_idx, n_heads, head_dim,
                                      budget.k_sink, budget.k_swa, pages, M, P, scores, ld_scores, RowGate{nullptr, 0},
                                      stream);
    return hip_status(e, "lsa_index_score launch");
}

int lsa_quantize_fp8(int dtype, int64_t n_vec, int32_t dim, const void *x, uint8_t *codes, float *scale,
                     hipStream_t stream)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (n_vec < 0 || dim < 1)
        return fail(LSA_ERR_INVALID, "n_vec >= 0 and dim >= 1 required");
    if (dim > 256)
        return fail(LSA_ERR_UNSUPPORTED, "dim above 256");
    if (n_vec >= ((int64_t)1 << 33))
        return fail(LSA_ERR_UNSUPPORTED, "n_vec too large");
    if (n_vec > 0 && (!x || !codes || !scale))
        return fail(LSA_ERR_INVALID, "x, codes and scale must be device pointers");
    hipError_t e = launch_quantize_fp8(dtype, n_vec, dim, x, codes, scale, stream);
    return hip_status(e, "lsa_quantize_fp8 launch");
}

int lsa_index_score_fp8(const lsa_rows_t *rows, const uint8_t *q8, const float *q_scale, const float *w,
                        const uint8_t *k8, const float *k_scale, int32_t n_heads, int32_t head_dim,
                        lsa_budget_t budget, const int32_t *pages, int32_t M, int32_t P, float *scores,
                        int64_t ld_scores, hipStream_t stream)
{
    if (int st = check_rows(rows))
        return st;
    if (int st = check_budget(budget))
        return st;
    if (n_heads != 64 || head_dim != 128)
        return fail(LSA_ERR_UNSUPPORTED, "FP8 indexer compiled for 64 heads of dim 128 only (got %d, %d)", n_heads,
                    head_dim);
    if (rows->n_rows > 0 && (!q8 || !q_scale || !w || !k8 || !k_scale || !scores))
        return fail(LSA_ERR_INVALID, "q8, q_scale, w, k8, k_scale and scores must be device pointers");
    if (pages) {
        if (M <= 0 || P <= 0)
            return fail(LSA_ERR_INVALID, "page mode needs M > 0 and P > 0");
        if (P % 16 != 0)
            return fail(LSA_ERR_UNSUPPORTED, "page mode needs P %% 16 == 0");
        if ((int64_t)M * P >= ((int64_t)1 << 31))
            return fail(LSA_ERR_INVALID, "M*P overflows int32");
        if (ld_scores < (int64_t)M * P)
            return fail(LSA_ERR_INVALID, "ld_scores %lld < M*P", (long long)ld_scores);
    } else if (ld_scores < rows->max_kv_len) {
        return fail(LSA_ERR_INVALID, "ld_scores %lld < max_kv_len %lld", (long long)ld_scores,
                    (long long)rows->max_kv_len);
    }
    if (ld_scores >= ((int64_t)1 << 31))
        return fail(LSA_ERR_UNSUPPORTED, "ld_scores must be below 2^31");
    hipError_t e = launch_index_score_fp8(to_dev(rows), q8, q_scale, w, k8, k_scale, budget.k_sink, budget.k_swa, pages,
                                          M, P, scores, ld_scores, stream);
    return hip_status(e, "lsa_index_score_fp8 launch");
}

// FP8 flat selection: the fused pass when rows x 8192-column chunks fill the chip, else the FP8 scores
// (first in the workspace) and the top-K levels over them.  (At 128K with 32 rows, a single round of
// 512 blocks, the fused pass still wins: 121.5 against 130.2 us for the separate passes.)
static bool fp8_fused(const lsa_rows_t *rows, int k)
{
    return k >= 1 && k <= 4096 && (int64_t)rows->n_rows * index_select_fused_segments(rows->max_kv_len) >= 256;
}

static size_t fp8_select_bytes(const lsa_rows_t *rows, int k, size_t *scores_bytes)
{
    const int64_t ld = rows->max_kv_len > 0 ? rows->max_kv_len : 1;
    if (fp8_fused(rows, k)) {
        *scores_bytes = 0;
        int64_t cols;
        return topk_lists_workspace_bytes(rows->n_rows, fp8_fused_segments(rows, ld, &cols), k);
    }
    *scores_bytes = align_up(sizeof(float) * (size_t)rows->n_rows * (size_t)ld);
    return *scores_bytes + topk_workspace_bytes(rows->n_rows, ld, k);
}

static int check_index_topk_fp8(const lsa_rows_t *rows, int32_t n_heads, int32_t head_dim, int32_t k)
{
    if (int st = check_rows(rows))
        return st;
    if (n_heads != 64 || head_dim != 128)
        return fail(LSA_ERR_UNSUPPORTED, "FP8 indexer compiled for 64 heads of dim 128 only (got %d, %d)", n_heads,
                    head_dim);
    if (k < 1 || k > 4096)
        return fail(LSA_ERR_UNSUPPORTED, "k_sparse must be in [1, 4096]");
    return LSA_OK;
}

int lsa_index_topk_fp8_workspace_size(const lsa_rows_t *rows, int32_t n_heads, int32_t head_dim, int32_t k_sparse,
                                      size_t *bytes)
{
    if (!bytes)
        return fail(LSA_ERR_INVALID, "bytes is NULL");
    if (int st = check_index_topk_fp8(rows, n_heads, head_dim, k_sparse))
        return st;
    size_t sb;
    *bytes = fp8_select_bytes(rows, k_sparse, &sb);
    return ok();
}

int lsa_index_topk_fp8(const lsa_rows_t *rows, const uint8_t *q8, const float *q_scale, const float *w,
                       const uint8_t *k8, const float *k_scale, int32_t n_heads, int32_t head_dim,
                       lsa_budget_t budget, int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (int st = check_index_topk_fp8(rows, n_heads, head_dim, budget.k_sparse))
        return st;
    if (int st = check_budget(budget))
        return st;
    if (rows->n_rows > 0 && (!q8 || !q_scale || !w || !k8 || !k_scale || !idx))
        return fail(LSA_ERR_INVALID, "q8, q_scale, w, k8, k_scale and idx must be device pointers");
    size_t sb;
    const size_t need = fp8_select_bytes(rows, budget.k_sparse, &sb);
    if (ws_bytes < need || (need && !ws))
        return fail(LSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
    if (ws && !aligned256(ws))
        return fail(LSA_ERR_INVALID, "workspace must be 256-byte aligned");
    if (rows->n_rows == 0)
        return ok();
    const RowsDev rd = to_dev(rows);
    const int64_t ld = rows->max_kv_len > 0 ? rows->max_kv_len : 1;
    const int k = budget.k_sparse;
    hipError_t e;
    if (fp8_fused(rows, k)) {
        int64_t cols;
        const int64_t n_seg = fp8_fused_segments(rows, ld, &cols);
        uint32_t *sk;
        int32_t *sp;
        int64_t sld;
        topk_first_lists(ws, rows->n_rows, n_seg, k, &sk, &sp, &sld);
        e = launch_index_select_fused_fp8(rd, q8, q_scale, w, k8, k_scale, budget.k_sink, budget.k_swa, ld, cols, k, sk,
                                          sp, sld, stream);
        if (e == hipSuccess)
            e = launch_topk_lists(rows->n_rows, n_seg, k, ws, idx, RowGate{nullptr, 0},
                                  ListCount{rd, budget.k_sink, budget.k_swa, cols, true}, stream);
    } else {
        float *scores = (float *)ws;
        e = launch_index_score_fp8(rd, q8, q_scale, w, k8, k_scale, budget.k_sink, budget.k_swa, nullptr, 0, 1, scores,
                                   ld, stream);
        if (e == hipSuccess)
            e = launch_topk(rows->n_rows, scores, ld, ld, nullptr, 0, 1, k, idx, (char *)ws + sb, RowGate{nullptr, 0},
                            stream);
    }
    return hip_status(e, "lsa_index_topk_fp8 launch");
}

int lsa_page_means(int dtype, int32_t n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                   int32_t head_dim, int32_t B, int64_t max_kv_len, int64_t first_token, void *k_mean,
                   hipStream_t stream)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (n_seq < 0 || head_dim <= 0 || B <= 0 || max_kv_len < 0 || first_token < 0)
        return fail(LSA_ERR_INVALID, "n_seq, head_dim, B, max_kv_len, first_token out of range");
    if (n_seq > kMaxGridRows)
        return fail(LSA_ERR_UNSUPPORTED, "n_seq above %lld", (long long)kMaxGridRows);
    if (n_seq > 0 && (!kv_off || !sb_off || !k_idx || !k_mean))
        return fail(LSA_ERR_INVALID, "kv_off, sb_off, k_idx and k_mean must be device pointers");
    if (ceil_div(max_kv_len, B) * head_dim >= ((int64_t)1 << 31) * 256)
        return fail(LSA_ERR_UNSUPPORTED, "too many sub-blocks");
    hipError_t e = launch_page_means(dtype, n_seq, kv_off, sb_off, k_idx, head_dim, B, max_kv_len, first_token, 0,
                                     k_mean, stream);
    return hip_status(e, "lsa_page_means launch");
}

int lsa_page_means_append(int dtype, int32_t n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                          int32_t head_dim, int32_t B, int64_t n_new, void *k_mean, hipStream_t stream)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (n_seq < 0 || head_dim <= 0 || B <= 0 || n_new < 1)
        return fail(LSA_ERR_INVALID, "n_seq, head_dim, B, n_new out of range");
    if (n_seq > kMaxGridRows)
        return fail(LSA_ERR_UNSUPPORTED, "n_seq above %lld", (long long)kMaxGridRows);
    if (n_seq > 0 && (!kv_off || !sb_off || !k_idx || !k_mean))
        return fail(LSA_ERR_INVALID, "kv_off, sb_off, k_idx and k_mean must be device pointers");
    if ((ceil_div(n_new, B) + 1) * head_dim >= ((int64_t)1 << 31) * 256)
        return fail(LSA_ERR_UNSUPPORTED, "n_new too large (use lsa_page_means)");
    // max_kv_len only gates the launch here: any value >= 1 lets every sequence through
    hipError_t e = launch_page_means(dtype, n_seq, kv_off, sb_off, k_idx, head_dim, B, 1, 0, n_new, k_mean, stream);
    return hip_status(e, "lsa_page_means_append launch");
}

int lsa_page_recall_workspace_size(const lsa_rows_t *rows, int32_t P, int32_t M, size_t *bytes)
{
    if (!bytes)
        return fail(LSA_ERR_INVALID, "bytes is NULL");
    if (int st = check_rows(rows))
        return st;
    if (P <= 0 || M <= 0)
        return fail(LSA_ERR_INVALID, "P and M must be positive");
    Carver c(nullptr);
    c.take(sizeof(float) * (size_t)rows->n_rows * (size_t)ceil_div(rows->max_kv_len, P));
    c.take(topk_workspace_bytes(rows->n_rows, ceil_div(rows->max_kv_len, P), M));
    *bytes = c.used;
    return ok();
}

int lsa_page_recall(int dtype, const lsa_rows_t *rows, const int64_t *sb_off, const void *q_idx, const float *w,
                    const void *k_mean, int32_t n_heads, int32_t head_dim, int32_t P, int32_t B, int32_t M,
                    float *page_scores, int64_t ld_ps, int32_t *pages, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (int st = check_rows(rows))
        return st;
    if (int st = check_page_geometry(dtype, P, B, M))
        return st;
    if (!index_score_supported(dtype, n_heads, head_dim))
        return fail(LSA_ERR_UNSUPPORTED, "indexer shape (%d heads, dim %d) not compiled for this dtype", n_heads,
                    head_dim);
    const int64_t n_pages = ceil_div(rows->max_kv_len, P);
    if (rows->n_rows > 0 && (!sb_off || !q_idx || !w || !k_mean || !pages))
        return fail(LSA_ERR_INVALID, "sb_off, q_idx, w, k_mean and pages must be device pointers");
    if (page_scores && ld_ps < n_pages)
        return fail(LSA_ERR_INVALID, "ld_ps %lld < ceil(max_kv_len / P) = %lld", (long long)ld_ps,
                    (long long)n_pages);
    size_t need = 0;
    lsa_page_recall_workspace_size(rows, P, M, &need);
    if (ws_bytes < need || (need && !ws))
        return fail(LSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
    if (ws && !aligned256(ws))
        return fail(LSA_ERR_INVALID, "workspace must be 256-byte aligned");
    Carver c(ws);
    float *ps_ws = (float *)c.take(sizeof(float) * (size_t)rows->n_rows * (size_t)n_pages);
    void *tk = c.take(topk_workspace_bytes(rows->n_rows, n_pages, M));
    float *ps = page_scores ? page_scores : ps_ws;
    int64_t ld = page_scores ? ld_ps : n_pages;
    if (n_pages == 0 || rows->n_rows == 0) {
        // nothing to rank: every slot empty
        hipError_t e = launch_topk(rows->n_rows, ps, ld > 0 ? ld : 1, 0, nullptr, 0, 1, M, pages, tk,
                                   RowGate{nullptr, 0}, stream);
        return hip_status(e, "lsa_page_recall launch");
    }
    RowsDev rd = to_dev(rows);
    hipError_t e = launch_page_scores(dtype, rd, rows->max_kv_len, sb_off, q_idx, w, k_mean, n_heads, head_dim, P, B,
                                      ps, ld, RowGate{nullptr, 0}, stream);
    if (e == hipSuccess)
        e = launch_topk(rows->n_rows, ps, ld, n_pages, nullptr, 0, 1, M, pages, tk, RowGate{nullptr, 0}, stream);
    return hip_status(e, "lsa_page_recall launch");
}

int lsa_topk_workspace_size(int32_t n_rows, int64_t n_cols, int32_t k, size_t *bytes)
{
    if (!bytes)
        return fail(LSA_ERR_INVALID, "bytes is NULL");
    if (n_rows < 0 || n_cols < 0 || k < 1)
        return fail(LSA_ERR_INVALID, "n_rows, n_cols >= 0 and k >= 1 required");
    *bytes = topk_workspace_bytes(n_rows, n_cols, k);
    return ok();
}

int lsa_topk(int32_t n_rows, const float *scores, int64_t ld_scores, int64_t n_cols, const int32_t *pages, int32_t M,
             int32_t P, int32_t k, int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (n_rows < 0 || n_cols < 0 || ld_scores < n_cols)
        return fail(LSA_ERR_INVALID, "need n_rows >= 0 and 0 <= n_cols <= ld_scores");
    if (n_rows > kMaxGridRows)
        return fail(LSA_ERR_UNSUPPORTED, "n_rows above %lld", (long long)kMaxGridRows);
    if (n_cols >= ((int64_t)1 << 31))
        return fail(LSA_ERR_UNSUPPORTED, "n_cols must be below 2^31");
    if (k < 1 || k > 4096)
        return fail(LSA_ERR_UNSUPPORTED, "k must be in [1, 4096]");
    if (pages) {
        if (M <= 0 || P <= 0)
            return fail(LSA_ERR_INVALID, "page map needs M > 0 and P > 0");
        if ((int64_t)M * P < n_cols)
            return fail(LSA_ERR_INVALID, "page map covers %lld columns < n_cols", (long long)M * P);
        if (P % 16 != 0)
            return fail(LSA_ERR_UNSUPPORTED, "page size P must be a multiple of 16");
    }
    if (n_rows > 0 && (!idx || (n_cols > 0 && !scores)))
        return fail(LSA_ERR_INVALID, "scores and idx must be device pointers");
    size_t need = topk_workspace_bytes(n_rows, n_cols, k);
    if (ws_bytes < need || (need && !ws))
        return fail(LSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
    if (ws && !aligned256(ws))
        return fail(LSA_ERR_INVALID, "workspace must be 256-byte aligned");
    hipError_t e = launch_topk(n_rows, scores, ld_scores > 0 ? ld_scores : 1, n_cols, pages, M, P, k, idx, ws,
                               RowGate{nullptr, 0}, stream);
    return hip_status(e, "lsa_topk launch");
}

int lsa_index_topk_workspace_size(int dtype, const lsa_rows_t *rows, int32_t n_heads, int32_t head_dim,
                                  int32_t k_sparse, size_t *bytes)
{
    if (!bytes)
        return fail(LSA_ERR_INVALID, "bytes is NULL");
    if (int st = check_index_topk(dtype, rows, n_heads, head_dim, k_sparse))
        return st;
    size_t sb;
    *bytes = flat_select_bytes(dtype, rows, n_heads, head_dim, k_sparse, &sb);
    return ok();
}

int lsa_index_topk(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                   int32_t n_heads, int32_t head_dim, lsa_budget_t budget, int32_t *idx, void *ws, size_t ws_bytes,
                   hipStream_t stream)
{
    size_t need;
    if (int st = lsa::index_topk_check(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, budget, idx, &need))
        return st;
    if (ws_bytes < need || (need && !ws))
        return fail(LSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
    if (ws && !aligned256(ws))
        return fail(LSA_ERR_INVALID, "workspace must be 256-byte aligned");
    if (rows->n_rows == 0)
        return ok();
    hipError_t e = launch_flat_select(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, budget, idx, ws,
                                      RowGate{nullptr, 0}, stream);
    return hip_status(e, "lsa_index_topk launch");
}

int lsa_hybrid_attn_workspace_size(int dtype, const lsa_rows_t *rows, int32_t n_heads, int32_t d_v,
                                   lsa_budget_t budget, size_t *bytes)
{
    if (!bytes)
        return fail(LSA_ERR_INVALID, "bytes is NULL");
    if (int st = check_rows(rows))
        return st;
    if (int st = check_budget(budget))
        return st;
    if (n_heads <= 0 || d_v <= 0)
        return fail(LSA_ERR_INVALID, "n_heads and d_v must be positive");
    *bytes = attn_workspace_bytes(dtype, rows->n_rows, n_heads, d_v,
                                  budget.k_sink + budget.k_swa + budget.k_sparse);
    return ok();
}

int lsa_hybrid_attn(int dtype, const lsa_rows_t *rows, const void *q, const void *kv, int32_t n_heads, int32_t d_qk,
                    int32_t d_v, float scale, lsa_budget_t budget, const int32_t *idx, const int32_t *idx_row,
                    void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (dtype != LSA_F32 && dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID, "dtype must be LSA_F32 or LSA_BF16");
    if (int st = check_rows(rows))
        return st;
    if (int st = check_budget(budget))
        return st;
    if (n_heads <= 0 || d_qk <= 0 || d_v <= 0)
        return fail(LSA_ERR_INVALID, "n_heads, d_qk and d_v must be positive");
    const int k_total = budget.k_sink + budget.k_swa + budget.k_sparse;
    if (!attn_supported(dtype, n_heads, d_qk, d_v, budget.k_sparse, k_total))
        return fail(LSA_ERR_UNSUPPORTED, "attention shape (H=%d, d_qk=%d, d_v=%d, K=%d) not compiled for this dtype",
                    n_heads, d_qk, d_v, k_total);
    if (rows->n_rows > 0 && (!q || !kv || !out || (budget.k_sparse > 0 && !idx)))
        return fail(LSA_ERR_INVALID, "q, kv, out (and idx when k_sparse > 0) must be device pointers");
    size_t need = attn_workspace_bytes(dtype, rows->n_rows, n_heads, d_v, k_total);
    if (ws_bytes < need || (need && !ws))
        return fail(LSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
    if (ws && !aligned256(ws))
        return fail(LSA_ERR_INVALID, "workspace must be 256-byte aligned");
    static const int32_t *kNoIdx = nullptr;
    hipError_t e = launch_hybrid_attn(dtype, to_dev(rows), q, kv, n_heads, d_qk, d_v, scale, budget.k_sink,
                                      budget.k_swa, budget.k_sparse, budget.k_sparse > 0 ? idx : kNoIdx, idx_row, out,
                                      lse, ws, stream);
    return hip_status(e, "lsa_hybrid_attn launch");
}

int lsa_layer_workspace_size(const lsa_layer_cfg_t *cfg, const lsa_rows_t *rows, int32_t use_hi, size_t *bytes)
{
    if (!bytes)
        return fail(LSA_ERR_INVALID, "bytes is NULL");
    if (int st = check_layer_cfg(cfg))
        return st;
    if (int st = check_rows(rows))
        return st;
    if (use_hi && cfg->is_owner)
        if (int st = check_page_geometry(cfg->dtype, cfg->P, cfg->B, cfg->M))
            return st;
    *bytes = layer_ws_layout(cfg, rows, use_hi && cfg->is_owner, nullptr).bytes;
    return ok();
}

int lsa_layer_fwd(const lsa_layer_cfg_t *cfg, const lsa_rows_t *rows, const int32_t *idx_row, const void *q_idx,
                  const float *w, const void *k_idx, const int64_t *sb_off, const void *k_mean, const void *q,
                  const void *kv, int32_t *idx, void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (int st = check_layer_cfg(cfg))
        return st;
    if (int st = check_rows(rows))
        return st;
    const bool owner = cfg->is_owner != 0;
    const bool use_hi = owner && k_mean != nullptr && cfg->hi_min_len <= rows->max_kv_len;
    if (use_hi) {
        if (int st = check_page_geometry(cfg->dtype, cfg->P, cfg->B, cfg->M))
            return st;
        if (!sb_off)
            return fail(LSA_ERR_INVALID, "HI needs sb_off with k_mean");
    }
    if (rows->n_rows > 0) {
        if (!q || !kv || !out || !idx)
            return fail(LSA_ERR_INVALID, "q, kv, out and idx must be device pointers");
        if (owner && (!q_idx || !w || !k_idx))
            return fail(LSA_ERR_INVALID, "the owner layer needs q_idx, w and k_idx");
    }
    if ((int64_t)rows->n_rows * rows->max_kv_len >= ((int64_t)1 << 40))
        return fail(LSA_ERR_UNSUPPORTED, "n_rows * max_kv_len too large");
    LayerWs lw = layer_ws_layout(cfg, rows, use_hi, nullptr);
    if (ws_bytes < lw.bytes || (lw.bytes && !ws))
        return fail(LSA_ERR_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, lw.bytes);
    if (ws && !aligned256(ws))
        return fail(LSA_ERR_INVALID, "workspace must be 256-byte aligned");
    lw = layer_ws_layout(cfg, rows, use_hi, ws);

    const RowsDev rd = to_dev(rows);
    const lsa_budget_t bud = cfg->budget;
    hipError_t e = hipSuccess;
    if (owner && rows->n_rows > 0) {
        // Row roles are only needed when rows can differ: with neither shared index rows nor a mix of
        // flat and HI rows (no HI, or every sequence at least hi_min_len long) the kernels run ungated,
        // and when every row takes HI the flat passes are not launched.
        const bool all_hi = use_hi && rows->min_kv_len >= cfg->hi_min_len;
        const bool need_modes = (use_hi && !all_hi) || idx_row != nullptr;
        if (need_modes)
            e = launch_row_modes(rd, idx_row, cfg->hi_min_len, use_hi ? 1 : 0, lw.row_mode, lw.row_lists,
                                 lw.row_counts, bud.k_sink, bud.k_swa, lw.fused_cols, lw.fused_table, lw.fused_cap,
                                 stream);
        const uint8_t *gate = need_modes ? lw.row_mode : nullptr;
        const int32_t *flat_list = need_modes ? lw.row_lists : nullptr;
        const int32_t *hi_list = need_modes ? lw.row_lists + rows->n_rows : nullptr;
        // Flat indexer rows ([paper] §2.2 Eq. 1-2 over mid(t)).
        if (e == hipSuccess && !all_hi)
            e = launch_flat_select(cfg->dtype, rows, q_idx, w, k_idx, cfg->n_heads_idx, cfg->head_dim_idx, bud, idx,
                                   lw.topk_ws,
                                   RowGate{gate, 1, flat_list, lw.row_counts, need_modes ? lw.fused_table : nullptr,
                                           lw.row_counts + 2},
                                   stream);
        if (use_hi) {
            // HI rows ([paper] §3.3): page recall, stage-2 scoring on the recalled pages, topK.
            const int64_t n_pages = ceil_div(rows->max_kv_len, cfg->P);
            const int64_t n_comp = (int64_t)cfg->M * cfg->P;
            if (e == hipSuccess)
                e = launch_page_scores(cfg->dtype, rd, rows->max_kv_len, sb_off, q_idx, w, k_mean, cfg->n_heads_idx,
                                       cfg->head_dim_idx, cfg->P, cfg->B, lw.page_scores, n_pages,
                                       RowGate{gate, 2}, stream);
            if (e == hipSuccess)
                e = launch_topk(rows->n_rows, lw.page_scores, n_pages, n_pages, nullptr, 0, 1, cfg->M, lw.pages,
                                lw.page_topk_ws, RowGate{gate, 2}, stream);
            if (e == hipSuccess)
                e = launch_index_score(cfg->dtype, rd, rows->max_kv_len, q_idx, w, k_idx, cfg->n_heads_idx,
                                       cfg->head_dim_idx, bud.k_sink, bud.k_swa, lw.pages, cfg->M, cfg->P,
                                       lw.comp_scores, n_comp, RowGate{gate, 2, hi_list, lw.row_counts + 1}, stream);
            if (e == hipSuccess)
                e = launch_topk(rows->n_rows, lw.comp_scores, n_comp, n_comp, lw.pages, cfg->M, cfg->P, bud.k_sparse,
                                idx, lw.topk_ws, RowGate{gate, 2}, stream);
        }
    }
    if (e == hipSuccess)
        e = launch_hybrid_attn(cfg->dtype, rd, q, kv, cfg->n_heads, cfg->d_qk, cfg->d_v, cfg->scale, bud.k_sink,
                               bud.k_swa, bud.k_sparse, idx, idx_row, out, lse, lw.attn_ws, stream);
    return hip_status(e, "lsa_layer_fwd launch");
}

}  // extern "C"
