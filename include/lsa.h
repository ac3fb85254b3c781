/*
 * lsa.h -- C ABI of the MI355X (gfx950) LongCat Sparse Attention layer-forward library, liblsa.
 *
 * One layer of LongCat Sparse Attention (LSA), forward only, on one GPU:
 *   Lightning-Indexer scoring, streaming-aware (SI) budget split, hierarchical (HI) page recall,
 *   arg-topK, and hybrid sparse attention over the MLA latent KV, with cross-layer (CLI) reuse.
 *
 * Pages cited below (titles as published):
 *   [paper]  "LongCat Sparse Attention: Taming the Lightning via Streaming-aware Hierarchical
 *            Cross-Layer Indexing" (arXiv 2608.01662)
 *   [review] "LongCat Sparse Attention：流式感知、分层与跨层索引协同设计" (Chinese-language review)
 *   [summary] the English summary page of the same paper ("Summary (Overview)")
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never allocates on
 *     these calls and never frees.  Scratch memory comes from a caller workspace whose size the
 *     matching lsa_*_workspace_size() returns (256-byte aligned pointer required).
 *   - Every call validates its scalars and host structs BEFORE any HIP call, enqueues its kernels
 *     on `stream` and returns without synchronising.  Results are bitwise deterministic.
 *   - Layouts are row-major, contiguous in the last dimension.  `dtype` is LSA_F32 or LSA_BF16
 *     for q_idx / k_idx / k_mean / q / kv / out; w, scores and lse are always fp32; positions and
 *     page indices are int32.
 *   - Positions are 0-indexed.  A query row r belongs to sequence b = row_seq[r], sits at
 *     position t = row_pos[r] and sees L_b = kv_off[b+1] - kv_off[b] cached tokens (t < L_b, the
 *     current token included).  Token s of sequence b is row kv_off[b] + s of k_idx / kv.
 *     With the budget (Ksink, Kswa, Ksparse) ([paper] §3.1, [review] §2.1):
 *         sink(t) = [0, min(Ksink, t+1))
 *         swa(t)  = [max(Ksink, t-Kswa+1), t]
 *         mid(t)  = [Ksink, t-Kswa]          (empty when t-Kswa < Ksink)
 *     A row with t < 0 or t >= L_b is treated as empty: no scores, no picks, out = 0, lse = -inf.
 *   - Return codes: LSA_OK, or an error code with a message in lsa_last_error() (thread-local).
 *     Invalid arguments -> LSA_ERR_INVALID; shapes no compiled kernel handles ->
 *     LSA_ERR_UNSUPPORTED; a workspace below the required size -> LSA_ERR_WORKSPACE; a failed HIP
 *     launch -> LSA_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Calls on one stream are ordered; calls that share a workspace must not overlap in time.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LSA_OK = 0, LSA_ERR_INVALID = 1, LSA_ERR_UNSUPPORTED = 2, LSA_ERR_WORKSPACE = 3, LSA_ERR_HIP = 4 };
enum { LSA_F32 = 0, LSA_BF16 = 1 };

/* Query rows of a batch of packed sequences (all device pointers except max_kv_len). */
typedef struct lsa_rows {
    int32_t n_seq;           /* number of sequences */
    int32_t n_rows;          /* number of query rows */
    const int64_t *kv_off;   /* device [n_seq+1]: token offsets, kv_off[0] = 0, non-decreasing */
    const int32_t *row_seq;  /* device [n_rows]: sequence of each row, in [0, n_seq) */
    const int32_t *row_pos;  /* device [n_rows]: position t of each row */
    int64_t max_kv_len;      /* host: an upper bound of every L_b; sizes grids and buffers */
    int64_t min_kv_len;      /* host: a lower bound of every L_b, or 0 when not known (0 <= min <= max);
                                used only to skip passes no row needs (lsa_layer_fwd: with
                                min_kv_len >= hi_min_len no row runs the flat indexer) */
} lsa_rows_t;

/* SI budget: K = k_sink + k_swa + k_sparse (the pages use 16 + 1024 + 1024, [paper] §3.1). */
typedef struct lsa_budget {
    int32_t k_sink, k_swa, k_sparse;
} lsa_budget_t;

/*
 * Lightning-Indexer scores ([paper] §2.2 Eq. 1; SI middle region [paper] §3.1, [review] §2.1):
 *     I(r, s) = sum_{j < n_heads} w[r, j] * ReLU(q_idx[r, j, :] . k_idx[kv_off[b] + s, :])
 * q_idx [n_rows, n_heads, head_dim]; w [n_rows, n_heads] fp32; k_idx [tokens, head_dim].
 *
 * Flat (pages == NULL): scores[r, s] for every s in [0, ld_scores) gets I(r, s) when
 *   s in mid(t) and s < L_b, else -inf.  Requires ld_scores >= rows->max_kv_len.
 * Page-mapped (HI stage 2, [paper] §3.3 "Token-level refinement"): pages [n_rows, M] lists
 *   recalled page indices (ascending, -1 = empty slot); column u in [0, M*P) stands for position
 *   pages[r, u/P]*P + u%P and gets its score when that position is in mid(t) and < L_b, else -inf;
 *   columns [M*P, ld_scores) get -inf.  Requires ld_scores >= M*P, P % 16 == 0.
 * Supported: fp32 with 1 <= n_heads <= 64 and head_dim 64 or 128; bf16 with
 *   (n_heads, head_dim) = (64, 128) on matrix cores.
 */
int lsa_index_score(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                    int32_t n_heads, int32_t head_dim, lsa_budget_t budget, const int32_t *pages, int32_t M,
                    int32_t P, float *scores, int64_t ld_scores, hipStream_t stream);

/*
 * FP8 form of the indexer inputs ([paper] §2.2 "Lightning Indexer": the indexer supports FP8
 * computation; the format below is this library's reading).  For each of the n_vec vectors of x
 * [n_vec, dim] (a key's d_I dims, or one query head): scale[v] = 2^e with e the smallest integer
 * such that max|x[v, :]| <= 448 * 2^e (e = 0 for an all-zero vector), and codes[v, i] = the OCP FP8
 * E4M3 code (bias 7, subnormals, no infinities) nearest to x[v, i] / 2^e, ties to the even code;
 * -0 is stored as +0 and no code saturates.  x is bf16 (dtype LSA_BF16) or fp32; codes [n_vec, dim]
 * uint8 and scale [n_vec] fp32 are device buffers owned by the caller.  1 <= dim <= 256.  A key
 * cache is quantized once, as tokens are appended; queries once per step.
 */
int lsa_quantize_fp8(int dtype, int64_t n_vec, int32_t dim, const void *x, uint8_t *codes, float *scale,
                     hipStream_t stream);

/*
 * Lightning-Indexer scores from FP8 inputs: Eq. 1 of lsa_index_score on the dequantized values
 *     I(r, s) = sum_j w[r, j] * ReLU(q_scale[r, j] * k_scale[s] * (dec(q8[r, j, :]) . dec(k8[s, :])))
 * with q8 [n_rows, n_heads, head_dim] / q_scale [n_rows, n_heads] and k8 [tokens, head_dim] /
 * k_scale [tokens] as produced by lsa_quantize_fp8; every other argument, the flat and page-mapped
 * column layouts, the -inf conventions and the errors are those of lsa_index_score.  Keys stream at
 * 132 bytes each instead of 256.  Supported: (n_heads, head_dim) = (64, 128), on the CDNA4 FP8
 * matrix instruction (products exact, sums in fp32).
 */
int lsa_index_score_fp8(const lsa_rows_t *rows, const uint8_t *q8, const float *q_scale, const float *w,
                        const uint8_t *k8, const float *k_scale, int32_t n_heads, int32_t head_dim,
                        lsa_budget_t budget, const int32_t *pages, int32_t M, int32_t P, float *scores,
                        int64_t ld_scores, hipStream_t stream);

/*
 * The FP8 flat selection in one call: idx [n_rows, budget.k_sparse] receives exactly what lsa_topk
 * (k = budget.k_sparse) returns for the flat scores of lsa_index_score_fp8 on the same inputs (pages ==
 * NULL), bit for bit.  When rows x 8192-column chunks fill the chip, each block keeps its chunk's scores
 * on chip and writes only its k best (score, position) pairs, as lsa_index_topk does for bf16.
 * Arguments and errors as for lsa_index_score_fp8 and lsa_index_topk; 1 <= k_sparse <= 4096.
 * Workspace: lsa_index_topk_fp8_workspace_size() bytes, 256-byte aligned.
 */
int lsa_index_topk_fp8(const lsa_rows_t *rows, const uint8_t *q8, const float *q_scale, const float *w,
                       const uint8_t *k8, const float *k_scale, int32_t n_heads, int32_t head_dim,
                       lsa_budget_t budget, int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream);
int lsa_index_topk_fp8_workspace_size(const lsa_rows_t *rows, int32_t n_heads, int32_t head_dim, int32_t k_sparse,
                                      size_t *bytes);

/*
 * Sub-block mean cache of the indexer keys ([paper] §3.3 "Design choices": precomputed once per
 * sequence and cached).  Sub-block n of sequence b covers tokens [nB, min((n+1)B, L_b)); row
 * sb_off[b] + n of k_mean [sb_off[n_seq], head_dim] receives the mean over the tokens present,
 * summed exactly in fp64 and rounded once to `dtype` (nearest-even).  sb_off [n_seq+1] (device)
 * must satisfy sb_off[b+1] - sb_off[b] = ceil(L_b / B).  first_token > 0 rebuilds only the
 * sub-blocks holding tokens >= first_token (the incremental update after appending tokens).
 * max_kv_len (host) bounds every L_b.
 */
int lsa_page_means(int dtype, int32_t n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                   int32_t head_dim, int32_t B, int64_t max_kv_len, int64_t first_token, void *k_mean,
                   hipStream_t stream);

/*
 * The per-step upkeep of the same cache ([paper] §3.3 "Design choices": the means are cached, so
 * each decode step only refreshes what the new tokens change): after every sequence b has grown by
 * n_new tokens (kv_off and sb_off already describe the new lengths L_b), rebuild the sub-blocks
 * holding tokens [max(L_b - n_new, 0), L_b) of each sequence -- at most ceil(n_new / B) + 1 per
 * sequence -- exactly as lsa_page_means would.  Rows of other sub-blocks are not touched.  The
 * launch covers n_new tokens per sequence whatever the lengths, so a decode step (n_new = 1) costs
 * one small launch.  Errors: LSA_ERR_INVALID for n_new < 1, a bad dtype or missing pointers.
 */
int lsa_page_means_append(int dtype, int32_t n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                          int32_t head_dim, int32_t B, int64_t n_new, void *k_mean, hipStream_t stream);

/*
 * HI stage 1 ([paper] §3.3 "Block-level coarse filtering"; recall set [review] §2.3):
 *   page score  S(r, p) = sum_j w[r,j] * sum_{n in page p} ReLU(q_idx[r,j,:] . k_mean[sb_off[b]+n,:])
 *   for the causal pages p <= floor(t / P) (-inf for the others), then pages[r, :M] = the M best
 *   pages under (score desc, page asc), listed ascending, -1 padded.
 * page_scores (nullable) [n_rows, ld_ps] receives the page scores (ld_ps >= ceil(max_kv_len/P));
 * when NULL they live in the workspace.  B must divide P and P / B <= 16.
 * Supported: the lsa_index_score shapes.  Workspace: lsa_page_recall_workspace_size().
 */
int lsa_page_recall(int dtype, const lsa_rows_t *rows, const int64_t *sb_off, const void *q_idx, const float *w,
                    const void *k_mean, int32_t n_heads, int32_t head_dim, int32_t P, int32_t B, int32_t M,
                    float *page_scores, int64_t ld_ps, int32_t *pages, void *ws, size_t ws_bytes,
                    hipStream_t stream);
int lsa_page_recall_workspace_size(const lsa_rows_t *rows, int32_t P, int32_t M, size_t *bytes);

/*
 * arg-topK ([paper] §2.2 Eq. 2; SI middle region [review] §2.1; HI stage 2 [paper] §3.3):
 * for each of n_rows rows of scores [n_rows, ld_scores], among the entries of columns [0, n_cols)
 * that are neither -inf nor NaN (+inf counts) take the k best under (score desc, position asc)
 * -- -0 equals +0 -- and write their positions ascending into idx [n_rows, k], padded with -1
 * when a row has fewer than k candidates.  pages == NULL: the position of column c is c.
 * Otherwise pages [n_rows, M] (ascending page lists, -1 = empty) maps column c to
 * pages[r, c/P]*P + c%P, and columns of empty slots are not candidates; P must be a multiple of
 * 16.  Limits: 1 <= k <= 4096, n_cols < 2^31.  Workspace: lsa_topk_workspace_size() bytes,
 * 256-byte aligned (may be NULL when that size is 0, i.e. n_cols <= 16384).
 */
int lsa_topk(int32_t n_rows, const float *scores, int64_t ld_scores, int64_t n_cols, const int32_t *pages,
             int32_t M, int32_t P, int32_t k, int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream);
int lsa_topk_workspace_size(int32_t n_rows, int64_t n_cols, int32_t k, size_t *bytes);

/*
 * The flat token selection in one call ([paper] §2.2 Eq. 1-2 over the SI middle region, [paper]
 * §3.1): idx [n_rows, budget.k_sparse] receives exactly what lsa_topk(k = budget.k_sparse) returns
 * for the flat scores of lsa_index_score (pages == NULL) -- the positions of the k_sparse best
 * mid(t) tokens under (score desc, position asc), ascending, -1 padded -- bit for bit.  When the
 * rows are scored one by one on matrix cores (bf16, 64 heads x 128 dims, fewer than 64 rows, enough
 * 8192-column chunks to fill the chip) scoring and the first top-K level run in one pass: each
 * block keeps its chunk's scores on chip and writes only its k best (score, position) pairs, so
 * the scores never reach HBM.  Otherwise the scores go through the workspace and lsa_topk.
 * Arguments, shapes, supported dtypes and errors are those of lsa_index_score and lsa_topk;
 * 1 <= k_sparse <= 4096.  Workspace: lsa_index_topk_workspace_size() bytes, 256-byte aligned.
 */
int lsa_index_topk(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                   int32_t n_heads, int32_t head_dim, lsa_budget_t budget, int32_t *idx, void *ws, size_t ws_bytes,
                   hipStream_t stream);
int lsa_index_topk_workspace_size(int dtype, const lsa_rows_t *rows, int32_t n_heads, int32_t head_dim,
                                  int32_t k_sparse, size_t *bytes);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, hosts that forbid hipMalloc): lsa_index_topk with its workspace in a device array of the
 * library, LSA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the first call on that GPU until
 * the process ends.  Same arguments, result and errors as lsa_index_topk minus (ws, ws_bytes);
 * rows whose lsa_index_topk_workspace_size() exceeds the array return LSA_ERR_UNSUPPORTED (64 MiB
 * holds the fused selection of 32 bf16 decode rows at 1M tokens).  The stream must belong to the
 * current device (else LSA_ERR_INVALID).  Allocates nothing.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (other streams, other host threads) race and must
 * be serialised by the caller.
 */
#define LSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lsa_index_topk_noalloc(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                           int32_t n_heads, int32_t head_dim, lsa_budget_t budget, int32_t *idx,
                           hipStream_t stream);

/*
 * Hybrid sparse attention over the MLA latent ([paper] §4.1.1 HFA; attention of [summary] "DSA
 * Mechanism Formalization"; latent layout [paper] §5.1 Table 6):
 *   S(r) = sink(t) u swa(t) u { idx[ir, i] : in mid(t), not equal to idx[ir, i-1] },
 *          ir = idx_row ? idx_row[r] : r   (CLI / MTP reuse, [paper] §3.2)
 *   for each head h:  z_s = scale * q[r,h,:] . kv[kv_off[b]+s, 0:d_qk]
 *                     out[r,h,:] = sum_s softmax(z)_s * kv[kv_off[b]+s, 0:d_v]
 *                     lse[r,h]   = log sum_s exp(z_s)        (natural log)
 * The contiguous sink+window rows and the gathered rows are processed as separate streams of
 * tiles and merged by online-softmax rescaling.  q [n_rows, n_heads, d_qk]; kv [tokens, d_qk];
 * idx [*, budget.k_sparse] ascending (as lsa_topk writes it); out [n_rows, n_heads, d_v] in
 * dtype; lse [n_rows, n_heads] fp32, nullable.
 * Supported: fp32 with d_qk <= 1024, d_v <= d_qk; bf16 with n_heads % 32 == 0, d_qk = 576, d_v = 512
 * on matrix cores.  Workspace: lsa_hybrid_attn_workspace_size().
 */
int lsa_hybrid_attn(int dtype, const lsa_rows_t *rows, const void *q, const void *kv, int32_t n_heads, int32_t d_qk,
                    int32_t d_v, float scale, lsa_budget_t budget, const int32_t *idx, const int32_t *idx_row,
                    void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);
int lsa_hybrid_attn_workspace_size(int dtype, const lsa_rows_t *rows, int32_t n_heads, int32_t d_v,
                                   lsa_budget_t budget, size_t *bytes);

/* Configuration of one LSA layer. */
typedef struct lsa_layer_cfg {
    int32_t dtype;        /* LSA_F32 or LSA_BF16 */
    int32_t n_heads_idx;  /* indexer heads H^I */
    int32_t head_dim_idx; /* indexer head dim d^I */
    int32_t n_heads;      /* attention heads */
    int32_t d_qk;         /* latent key dim (512 + 64 = 576) */
    int32_t d_v;          /* latent value dim (512) */
    float scale;          /* softmax scale */
    lsa_budget_t budget;  /* Ksink, Kswa, Ksparse */
    int32_t P, B, M;      /* HI page size, sub-block size, recalled pages */
    int64_t hi_min_len;   /* sequences with L_b >= hi_min_len use HI (INT64_MAX: never) */
    int32_t is_owner;     /* 1: indexer + topK + attention, writes idx; 0 (CLI reuse): attention with idx */
} lsa_layer_cfg_t;

/*
 * One LSA layer forward ([paper] §3: SI + CLI + HI; §4.1).
 * Owner layer: each index-owner row r (idx_row == NULL or idx_row[r] == r) runs the indexer on
 *   mid(t) -- flat, or HI (page recall, stage-2 scoring, topK) when k_mean != NULL and
 *   L_b >= hi_min_len -- and writes idx[r, :Ksparse]; rows that are not index owners keep their
 *   idx row untouched.  Reuse layer (is_owner = 0): idx is read, q_idx / w / k_idx are unused
 *   ([paper] §3.2; §4.1: reuse needs no kernel change).
 * Every row then attends over S(r) with index row idx_row[r] (MTP drafts: [paper] §3.2).
 * q_idx [n_rows, H^I, d^I]; w [n_rows, H^I]; k_idx [tokens, d^I]; sb_off / k_mean as written by
 * lsa_page_means (B = cfg->B), nullable when HI is off; q / kv / out / lse as lsa_hybrid_attn;
 * idx [n_rows, Ksparse].  Workspace: lsa_layer_workspace_size().
 */
int lsa_layer_fwd(const lsa_layer_cfg_t *cfg, const lsa_rows_t *rows, const int32_t *idx_row, const void *q_idx,
                  const float *w, const void *k_idx, const int64_t *sb_off, const void *k_mean, const void *q,
                  const void *kv, int32_t *idx, void *out, float *lse, void *ws, size_t ws_bytes,
                  hipStream_t stream);
int lsa_layer_workspace_size(const lsa_layer_cfg_t *cfg, const lsa_rows_t *rows, int32_t use_hi, size_t *bytes);

/* Status text of a return code, and the last error message of the calling thread. */
const char *lsa_status_string(int status);
const char *lsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
