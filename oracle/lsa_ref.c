/*
 * lsa_ref.c -- the CPU oracle for one LongCat Sparse Attention (LSA) layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct definition that the
 * HIP library is checked against.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it.  It shares no code, header, table or helper with the HIP library.
 *
 * Arithmetic: every bf16 / fp32 input decodes exactly into a double; all sums are fp64 in index
 * order; each result is rounded once to its output type (fp32 by the C cast, bf16 by
 * round-to-nearest-even from the double).
 *
 * Pages cited (titles as published):
 *   [paper]   "LongCat Sparse Attention: Taming the Lightning via Streaming-aware Hierarchical
 *             Cross-Layer Indexing" (arXiv 2608.01662, markdown rendering of the full paper)
 *   [review]  "LongCat Sparse Attention：流式感知、分层与跨层索引协同设计" (Chinese-language review)
 *   [summary] the English summary page of the same paper ("Summary (Overview)")
 *
 * Positions are 0-indexed here; the pages count from 1.  For a query row at position t of a
 * sequence of L cached tokens (t < L, the current token included):
 *   sink(t) = [0, min(Ksink, t+1))
 *   swa(t)  = [max(Ksink, t-Kswa+1), t]
 *   mid(t)  = [Ksink, t-Kswa]            (empty when t-Kswa < Ksink)
 * The three ranges are disjoint and cover [0, t].
 *
 * Parity pins: every function below is pinned by tests/test_oracle_*.py against closed forms,
 * special cases that reduce to textbook routines (dense softmax attention, a full sort) and
 * brute force on tiny inputs.  No function here is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_F32 0
#define REF_BF16 1

/* ------------------------------------------------------------------ scalar conversions */

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(int dtype, const void *base, int64_t i)
{
    if (dtype == REF_BF16)
        return bf16_bits_to_double(((const uint16_t *)base)[i]);
    return (double)((const float *)base)[i];
}

/* Round a double to the nearest bf16 (ties to even) in one step. */
static uint16_t double_to_bf16_bits(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return 0x7FC0u;
    double ax = fabs(x);
    if (isinf(ax))
        return sign | 0x7F80u;
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);            /* ax in [2^(e-1), 2^e) */
    int q = e - 8;            /* bf16 keeps 8 significant bits: spacing 2^(e-8) */
    if (q < -133)             /* below the normal range the spacing stays 2^-133 */
        q = -133;
    double r = nearbyint(ldexp(ax, -q)); /* default rounding mode: to nearest, ties to even */
    double v = ldexp(r, q);
    if (v >= 0x1p128)
        return sign | 0x7F80u;
    float f = (float)v; /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

static void store_elem(int dtype, void *base, int64_t i, double v)
{
    if (dtype == REF_BF16)
        ((uint16_t *)base)[i] = double_to_bf16_bits(v);
    else
        ((float *)base)[i] = (float)v;
}

/* Exposed so the tests can pin the rounding itself. */
uint16_t lsa_ref_double_to_bf16(double x) { return double_to_bf16_bits(x); }

/* ------------------------------------------------------------------ row-parallel driver */

typedef void (*row_fn)(void *ctx, int64_t row);

typedef struct {
    row_fn fn;
    void *ctx;
    int64_t n;
    int64_t next; /* shared work counter */
} pool_t;

static void *pool_worker(void *arg)
{
    pool_t *p = (pool_t *)arg;
    for (;;) {
        int64_t r = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
        if (r >= p->n)
            break;
        p->fn(p->ctx, r);
    }
    return NULL;
}

/* Runs fn(ctx, r) for r in [0, n) on up to n_threads threads (rows are independent). */
static void parallel_rows(row_fn fn, void *ctx, int64_t n, int n_threads)
{
    pool_t p = {fn, ctx, n, 0};
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if (n_threads == 1 || n <= 1) {
        pool_worker(&p);
        return;
    }
    pthread_t th[256];
    int started = 0;
    for (int i = 0; i < n_threads - 1; ++i)
        if (pthread_create(&th[started], NULL, pool_worker, &p) == 0)
            ++started;
    pool_worker(&p);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------ a1: streaming-aware ranges */

/*
 * [paper] §3.1 "Streaming-aware budget partitioning" and [review] §2.1: the budget is the union
 * of a sink of the first Ksink tokens, a sliding window of the last Kswa tokens ending at t, and
 * Ksparse tokens chosen by the indexer from the rest; the three parts are mutually exclusive.
 * For small t the window is clipped so that it never overlaps the sink.
 * out[0..1] = sink, out[2..3] = swa, out[4..5] = mid, each half-open [lo, hi) with lo <= hi.
 * A row outside its sequence (t < 0 or t >= L) gets three empty ranges.
 */
void lsa_ref_ranges(int64_t t, int64_t L, int64_t k_sink, int64_t k_swa, int64_t out[6])
{
    if (t < 0 || t >= L) {
        for (int i = 0; i < 6; ++i)
            out[i] = 0;
        return;
    }
    int64_t sink_hi = k_sink < t + 1 ? k_sink : t + 1;
    int64_t swa_lo = t - k_swa + 1;
    if (swa_lo < k_sink)
        swa_lo = k_sink;
    int64_t swa_hi = t + 1;
    if (swa_lo > swa_hi)
        swa_lo = swa_hi;
    int64_t mid_lo = k_sink;
    int64_t mid_hi = t - k_swa + 1;
    if (mid_hi < mid_lo)
        mid_hi = mid_lo;
    out[0] = 0;
    out[1] = sink_hi;
    out[2] = swa_lo;
    out[3] = swa_hi;
    out[4] = mid_lo;
    out[5] = mid_hi;
}

/* ------------------------------------------------------------------ a2: Lightning Indexer score */

/*
 * [paper] §2.2 "Indexer scoring" (Eq. 1): I(t,s) = sum over indexer heads j of
 * w(t,j) * ReLU(q(t,j) . k(s)), with one key shared by all heads (MQA).  No scale, no softmax.
 * q_row: [HI, dI]; w_row: [HI] fp32; k_vec: [dI].
 */
double lsa_ref_score_one(int dtype, const void *q_row, const float *w_row, const void *k_vec,
                         int HI, int dI)
{
    double acc = 0.0;
    for (int j = 0; j < HI; ++j) {
        double dot = 0.0;
        for (int d = 0; d < dI; ++d)
            dot += load_elem(dtype, q_row, (int64_t)j * dI + d) * load_elem(dtype, k_vec, d);
        double relu = dot > 0.0 ? dot : 0.0;
        acc += (double)w_row[j] * relu;
    }
    return acc;
}

typedef struct {
    int dtype;
    const int64_t *kv_off;
    const int32_t *row_seq, *row_pos;
    const void *q_idx;
    const float *w;
    const void *k_idx;
    int HI, dI;
    int64_t k_sink, k_swa;
    const int32_t *pages; /* NULL: flat columns are positions */
    int64_t M, P;
    float *scores;
    int64_t ld;
    const int32_t *only; /* NULL, or per-row flag: nonzero rows are scored, others left alone */
} score_ctx;

static int64_t elem_size(int dtype) { return dtype == REF_BF16 ? 2 : 4; }

static void score_row(void *vctx, int64_t r)
{
    const score_ctx *c = (const score_ctx *)vctx;
    if (c->only && !c->only[r])
        return;
    int64_t b = c->row_seq[r];
    int64_t base = c->kv_off[b];
    int64_t L = c->kv_off[b + 1] - base;
    int64_t t = c->row_pos[r];
    int64_t rg[6];
    lsa_ref_ranges(t, L, c->k_sink, c->k_swa, rg);
    const char *q_row = (const char *)c->q_idx + r * (int64_t)c->HI * c->dI * elem_size(c->dtype);
    const float *w_row = c->w + r * (int64_t)c->HI;
    float *out = c->scores + r * c->ld;
    for (int64_t col = 0; col < c->ld; ++col) {
        int64_t s = col;
        if (c->pages) {
            /* [paper] §3.3 "Stage 2: Token-level refinement": only tokens of recalled pages */
            if (col >= c->M * c->P) {
                out[col] = -INFINITY;
                continue;
            }
            int64_t pg = c->pages[r * c->M + col / c->P];
            s = pg < 0 ? -1 : pg * c->P + col % c->P;
        }
        /* SI: the indexer scores only the middle region ([paper] §3.1, [review] §2.1). */
        if (s < rg[4] || s >= rg[5] || s >= L) {
            out[col] = -INFINITY;
            continue;
        }
        const char *k_vec = (const char *)c->k_idx + (base + s) * (int64_t)c->dI * elem_size(c->dtype);
        out[col] = (float)lsa_ref_score_one(c->dtype, q_row, w_row, k_vec, c->HI, c->dI);
    }
}

/*
 * Flat (pages == NULL): scores[r, s] for s in [0, ld) = I(t_r, s) if s in mid(t_r), else -inf.
 * Page-mapped: column u in [0, M*P) stands for position pages[r, u/P]*P + u%P; -inf where the
 * page slot is -1 or the position is outside mid(t_r) or beyond the sequence.
 */
void lsa_ref_index_score(int dtype, const int64_t *kv_off, int n_rows, const int32_t *row_seq,
                         const int32_t *row_pos, const void *q_idx, const float *w, const void *k_idx,
                         int HI, int dI, int64_t k_sink, int64_t k_swa, const int32_t *pages, int64_t M,
                         int64_t P, float *scores, int64_t ld, const int32_t *only, int n_threads)
{
    score_ctx c = {dtype, kv_off, row_seq, row_pos, q_idx, w, k_idx, HI, dI, k_sink, k_swa,
                   pages, M, P, scores, ld, only};
    parallel_rows(score_row, &c, n_rows, n_threads);
}

/* ------------------------------------------------------------------ a7: arg-topK */

typedef struct {
    float score;
    int64_t pos;
} cand_t;

/* Total order of [paper] §2.2 Eq. 2 with the tie rule of lower position first. */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->score > y->score)
        return -1;
    if (x->score < y->score)
        return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int pos_cmp(const void *a, const void *b)
{
    int64_t x = ((const cand_t *)a)->pos, y = ((const cand_t *)b)->pos;
    return (x > y) - (x < y);
}

/*
 * Select the K best finite entries of one row (score descending, position ascending on ties;
 * -0 == +0 by value), list their positions ascending, pad with -1.  Returns the number selected,
 * or -1 if the row holds a NaN (undefined input).
 */
static int64_t topk_row(const float *row, int64_t n_cols, const int32_t *page_row, int64_t P, int64_t K,
                        int32_t *out, cand_t *buf)
{
    int64_t n = 0;
    for (int64_t c = 0; c < n_cols; ++c) {
        float v = row[c];
        if (isnan(v))
            return -1;
        if (isinf(v) && v < 0)
            continue;
        int64_t pos = c;
        if (page_row) {
            int64_t pg = page_row[c / P];
            if (pg < 0)
                continue;
            pos = pg * P + c % P;
        }
        buf[n].score = v;
        buf[n].pos = pos;
        ++n;
    }
    qsort(buf, (size_t)n, sizeof(cand_t), cand_cmp);
    int64_t take = n < K ? n : K;
    qsort(buf, (size_t)take, sizeof(cand_t), pos_cmp);
    for (int64_t i = 0; i < K; ++i)
        out[i] = i < take ? (int32_t)buf[i].pos : -1;
    return take;
}

typedef struct {
    const float *scores;
    int64_t ld, n_cols;
    const int32_t *pages;
    int64_t M, P, K;
    int32_t *idx;
    const int32_t *only;
    int status;
} topk_ctx;

static void topk_rowfn(void *vctx, int64_t r)
{
    topk_ctx *c = (topk_ctx *)vctx;
    if (c->only && !c->only[r])
        return;
    cand_t *buf = (cand_t *)malloc(sizeof(cand_t) * (size_t)(c->n_cols > 0 ? c->n_cols : 1));
    if (!buf) {
        c->status = -2;
        return;
    }
    int64_t got = topk_row(c->scores + r * c->ld, c->n_cols, c->pages ? c->pages + r * c->M : NULL,
                           c->P, c->K, c->idx + r * c->K, buf);
    if (got < 0)
        c->status = -1;
    free(buf);
}

/*
 * [paper] §2.2 Eq. 2 (arg-topK), restricted by SI to the middle region ([review] §2.1, S_sparse)
 * and, under HI, to the recalled pages ([paper] §3.3, Stage 2).  idx: [n_rows, K].
 * Returns 0, or -1 if a NaN score was seen.
 */
int lsa_ref_topk(const float *scores, int n_rows, int64_t ld, int64_t n_cols, const int32_t *pages,
                 int64_t M, int64_t P, int64_t K, int32_t *idx, const int32_t *only, int n_threads)
{
    topk_ctx c = {scores, ld, n_cols, pages, M, P, K, idx, only, 0};
    parallel_rows(topk_rowfn, &c, n_rows, n_threads);
    return c.status;
}

/* ------------------------------------------------------------------ a3: sub-block mean cache */

/*
 * [paper] §3.3 "Stage 1" and "Design choices": each page of P tokens is split into sub-blocks of
 * B tokens whose mean key is precomputed once per sequence and cached.  Sub-block n of sequence b
 * covers tokens [nB, min((n+1)B, L_b)); its mean is over the tokens present.  Row sb_off[b] + n of
 * k_mean holds it, rounded once to the storage dtype.  Returns -1 if sb_off is inconsistent.
 */
int lsa_ref_page_means(int dtype, int n_seq, const int64_t *kv_off, const int64_t *sb_off,
                       const void *k_idx, int dI, int64_t B, void *k_mean)
{
    for (int b = 0; b < n_seq; ++b) {
        int64_t L = kv_off[b + 1] - kv_off[b];
        int64_t nsb = (L + B - 1) / B;
        if (sb_off[b + 1] - sb_off[b] != nsb)
            return -1;
        for (int64_t n = 0; n < nsb; ++n) {
            int64_t lo = n * B, hi = (n + 1) * B < L ? (n + 1) * B : L;
            for (int d = 0; d < dI; ++d) {
                double sum = 0.0;
                for (int64_t s = lo; s < hi; ++s)
                    sum += load_elem(dtype, k_idx, (kv_off[b] + s) * dI + d);
                store_elem(dtype, k_mean, (sb_off[b] + n) * dI + d, sum / (double)(hi - lo));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ a4/a5: page score + recall */

typedef struct {
    int dtype;
    const int64_t *kv_off, *sb_off;
    const int32_t *row_seq, *row_pos;
    const void *q_idx;
    const float *w;
    const void *k_mean;
    int HI, dI;
    int64_t P, B;
    float *page_scores;
    int64_t ld;
    const int32_t *only;
} page_ctx;

static void page_row(void *vctx, int64_t r)
{
    const page_ctx *c = (const page_ctx *)vctx;
    if (c->only && !c->only[r])
        return;
    int64_t b = c->row_seq[r];
    int64_t L = c->kv_off[b + 1] - c->kv_off[b];
    int64_t t = c->row_pos[r];
    int64_t nsb = c->sb_off[b + 1] - c->sb_off[b];
    int64_t n_pages = (L + c->P - 1) / c->P;
    int64_t per_page = c->P / c->B;
    const char *q_row = (const char *)c->q_idx + r * (int64_t)c->HI * c->dI * elem_size(c->dtype);
    const float *w_row = c->w + r * (int64_t)c->HI;
    float *out = c->page_scores + r * c->ld;
    for (int64_t p = 0; p < c->ld; ++p) {
        /* [review] §2.3: pages compete for recall when p <= ceil(t/P) in 1-indexed terms, i.e.
         * 0-indexed page p <= floor(t/P), the page holding t and every earlier one. */
        if (t < 0 || t >= L || p > t / c->P || p >= n_pages) {
            out[p] = -INFINITY;
            continue;
        }
        /* [paper] §3.3 Stage 1 (page score): sum_j w_j * sum_{n in page p} ReLU(q_j . kmean_n) */
        double acc = 0.0;
        for (int j = 0; j < c->HI; ++j) {
            double inner = 0.0;
            for (int64_t n = p * per_page; n < (p + 1) * per_page && n < nsb; ++n) {
                double dot = 0.0;
                for (int d = 0; d < c->dI; ++d)
                    dot += load_elem(c->dtype, q_row, (int64_t)j * c->dI + d) *
                           load_elem(c->dtype, c->k_mean, (c->sb_off[b] + n) * c->dI + d);
                inner += dot > 0.0 ? dot : 0.0;
            }
            acc += (double)w_row[j] * inner;
        }
        out[p] = (float)acc;
    }
}

/* page_scores[r, p] for p in [0, ld): the stage-1 score of eligible pages, -inf otherwise. */
void lsa_ref_page_scores(int dtype, const int64_t *kv_off, const int64_t *sb_off, int n_rows,
                         const int32_t *row_seq, const int32_t *row_pos, const void *q_idx, const float *w,
                         const void *k_mean, int HI, int dI, int64_t P, int64_t B, float *page_scores,
                         int64_t ld, const int32_t *only, int n_threads)
{
    page_ctx c = {dtype, kv_off, sb_off, row_seq, row_pos, q_idx, w, k_mean, HI, dI, P, B,
                  page_scores, ld, only};
    parallel_rows(page_row, &c, n_rows, n_threads);
}

/*
 * [review] §2.3: P_t = arg-topK of the page scores over eligible pages, M of them.  The recalled
 * pages are listed ascending and padded with -1 (pages: [n_rows, M]).  Ties go to the lower page.
 * ws_scores must hold n_rows * ld floats; ld >= the largest page count of any sequence.
 */
int lsa_ref_page_recall(int dtype, const int64_t *kv_off, const int64_t *sb_off, int n_rows,
                        const int32_t *row_seq, const int32_t *row_pos, const void *q_idx, const float *w,
                        const void *k_mean, int HI, int dI, int64_t P, int64_t B, int64_t M, float *ws_scores,
                        int64_t ld, int32_t *pages, const int32_t *only, int n_threads)
{
    lsa_ref_page_scores(dtype, kv_off, sb_off, n_rows, row_seq, row_pos, q_idx, w, k_mean, HI, dI, P, B,
                        ws_scores, ld, only, n_threads);
    return lsa_ref_topk(ws_scores, n_rows, ld, ld, NULL, 0, 1, M, pages, only, n_threads);
}

/* ------------------------------------------------------------------ a8-a10: sparse attention */

typedef struct {
    int dtype;
    const int64_t *kv_off;
    const int32_t *row_seq, *row_pos;
    const void *q, *kv;
    int H, Dqk, Dv;
    double scale;
    int64_t k_sink, k_swa, k_sparse;
    const int32_t *idx, *idx_row;
    void *out;
    float *lse;
    int status;
} attn_ctx;

static int i64_cmp(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* The selected set S_t as ascending positions; returns |S_t|.  set must hold Ksink+Kswa+Ksparse. */
static int64_t selected_set(const attn_ctx *c, int64_t r, int64_t *set)
{
    int64_t b = c->row_seq[r];
    int64_t L = c->kv_off[b + 1] - c->kv_off[b];
    int64_t t = c->row_pos[r];
    int64_t rg[6];
    lsa_ref_ranges(t, L, c->k_sink, c->k_swa, rg);
    int64_t n = 0;
    for (int64_t s = rg[0]; s < rg[1]; ++s)
        set[n++] = s;
    int64_t ir = c->idx_row ? c->idx_row[r] : r;
    /* Only indexer picks that lie in mid(t) belong to S_sparse; repeats count once (a set). */
    int64_t n0 = n;
    for (int64_t i = 0; i < c->k_sparse; ++i) {
        int64_t s = c->idx[ir * c->k_sparse + i];
        if (s >= rg[4] && s < rg[5])
            set[n++] = s;
    }
    qsort(set + n0, (size_t)(n - n0), sizeof(int64_t), i64_cmp);
    int64_t m = n0;
    for (int64_t i = n0; i < n; ++i)
        if (i == n0 || set[i] != set[i - 1])
            set[m++] = set[i];
    n = m;
    for (int64_t s = rg[2]; s < rg[3]; ++s)
        set[n++] = s;
    qsort(set, (size_t)n, sizeof(int64_t), i64_cmp);
    return n;
}

static void attn_row(void *vctx, int64_t r)
{
    attn_ctx *c = (attn_ctx *)vctx;
    int64_t cap = c->k_sink + c->k_swa + c->k_sparse + 1;
    int64_t *set = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    double *z = (double *)malloc(sizeof(double) * (size_t)cap);
    double *o = (double *)malloc(sizeof(double) * (size_t)c->Dv);
    if (!set || !z || !o) {
        c->status = -2;
        free(set), free(z), free(o);
        return;
    }
    int64_t n = selected_set(c, r, set);
    int64_t base = c->kv_off[c->row_seq[r]];
    int64_t es = elem_size(c->dtype);
    for (int h = 0; h < c->H; ++h) {
        const char *qh = (const char *)c->q + ((int64_t)r * c->H + h) * c->Dqk * es;
        int64_t out_off = ((int64_t)r * c->H + h) * c->Dv;
        if (n == 0) {
            for (int d = 0; d < c->Dv; ++d)
                store_elem(c->dtype, c->out, out_off + d, 0.0);
            if (c->lse)
                c->lse[(int64_t)r * c->H + h] = -INFINITY;
            continue;
        }
        /* [summary] "DSA Mechanism Formalization": u_t = Attn(h_t, {c_s : s in S_t}).  On the MLA
         * latent the key is the full 576-dim row (512 latent + 64 RoPE) and the value is its first
         * 512 dims ([paper] §5.1 Table 6: kv rank 512, rope 64; §2.3: 1,152 B per row). */
        double mx = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            const char *kr = (const char *)c->kv + (base + set[i]) * (int64_t)c->Dqk * es;
            double dot = 0.0;
            for (int d = 0; d < c->Dqk; ++d)
                dot += load_elem(c->dtype, qh, d) * load_elem(c->dtype, kr, d);
            z[i] = c->scale * dot;
            if (z[i] > mx)
                mx = z[i];
        }
        double l = 0.0;
        for (int d = 0; d < c->Dv; ++d)
            o[d] = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double p = exp(z[i] - mx);
            l += p;
            const char *vr = (const char *)c->kv + (base + set[i]) * (int64_t)c->Dqk * es;
            for (int d = 0; d < c->Dv; ++d)
                o[d] += p * load_elem(c->dtype, vr, d);
        }
        for (int d = 0; d < c->Dv; ++d)
            store_elem(c->dtype, c->out, out_off + d, o[d] / l);
        if (c->lse)
            c->lse[(int64_t)r * c->H + h] = (float)(mx + log(l));
    }
    free(set), free(z), free(o);
}

/*
 * Softmax attention of each query head over S_t = sink(t) u swa(t) u (idx row & mid(t)).
 * [paper] §4.1.1 splits this into a contiguous (sink+window) branch and a gathered branch merged
 * by online-softmax rescaling; that split is an identity of the softmax, so the oracle computes
 * the union directly in two passes (max, then exp-sums).  q: [n_rows, H, Dqk]; kv: [tokens, Dqk];
 * out: [n_rows, H, Dv]; lse: [n_rows, H] (natural log of the softmax denominator, scale included).
 * idx_row (nullable): row r uses index row idx_row[r] (cross-layer / MTP reuse, [paper] §3.2).
 */
int lsa_ref_hybrid_attn(int dtype, const int64_t *kv_off, int n_rows, const int32_t *row_seq,
                        const int32_t *row_pos, const void *q, const void *kv, int H, int Dqk, int Dv,
                        double scale, int64_t k_sink, int64_t k_swa, int64_t k_sparse, const int32_t *idx,
                        const int32_t *idx_row, void *out, float *lse, int n_threads)
{
    attn_ctx c = {dtype, kv_off, row_seq, row_pos, q, kv, H, Dqk, Dv, scale, k_sink, k_swa, k_sparse,
                  idx, idx_row, out, lse, 0};
    parallel_rows(attn_row, &c, n_rows, n_threads);
    return c.status;
}

/* S_t of one row as ascending positions (for invariant checks); returns |S_t|. */
int64_t lsa_ref_selected_set(const int64_t *kv_off, const int32_t *row_seq, const int32_t *row_pos,
                             int64_t k_sink, int64_t k_swa, int64_t k_sparse, const int32_t *idx,
                             const int32_t *idx_row, int64_t r, int64_t *set_out)
{
    attn_ctx c;
    memset(&c, 0, sizeof c);
    c.kv_off = kv_off;
    c.row_seq = row_seq;
    c.row_pos = row_pos;
    c.k_sink = k_sink;
    c.k_swa = k_swa;
    c.k_sparse = k_sparse;
    c.idx = idx;
    c.idx_row = idx_row;
    return selected_set(&c, r, set_out);
}

/* ------------------------------------------------------------------ a11/a12: one layer */

/*
 * One LSA layer forward.
 *  - Owner layer (is_owner = 1): every index-owner row r (idx_row == NULL or idx_row[r] == r)
 *    runs the indexer on mid(t_r) and writes idx[r, :Ksparse].  Rows of a sequence with
 *    L >= hi_min_len use Hierarchical Indexing ([paper] §3.3, enabled adaptively beyond the
 *    crossover; §4.1.2): page recall of M pages, Eq. 1 on the recalled tokens, topK over them.
 *  - Reuse layer (is_owner = 0): the owner's idx is read, no indexer runs ([paper] §3.2, §4.1:
 *    cross-layer reuse needs no kernel change).
 *  - Every row then attends over S_t with index row idx_row[r] (MTP drafts share the index of
 *    their sequence's first query, [paper] §3.2 "Integration with Multi-Token Prediction").
 * Work buffers: flat_ws [n_rows, max_len] fp32, page_ws [n_rows, max_pages] fp32, pages_ws
 * [n_rows, M] int32, comp_ws [n_rows, M*P] fp32 (the HI ones may be NULL when HI is never used).
 */
int lsa_ref_layer_fwd(int dtype, int HI, int dI, int H, int Dqk, int Dv, double scale, int64_t k_sink,
                      int64_t k_swa, int64_t k_sparse, int64_t P, int64_t B, int64_t M, int64_t hi_min_len,
                      int is_owner, int n_seq, const int64_t *kv_off, int n_rows, const int32_t *row_seq,
                      const int32_t *row_pos, const int32_t *idx_row, const void *q_idx, const float *w,
                      const void *k_idx, const int64_t *sb_off, const void *k_mean, const void *q,
                      const void *kv, int32_t *idx, void *out, float *lse, float *flat_ws, int64_t max_len,
                      float *page_ws, int64_t max_pages, int32_t *pages_ws, float *comp_ws, int n_threads)
{
    if (is_owner) {
        int32_t *flat_rows = (int32_t *)calloc((size_t)n_rows + 1, sizeof(int32_t));
        int32_t *hi_rows = (int32_t *)calloc((size_t)n_rows + 1, sizeof(int32_t));
        if (!flat_rows || !hi_rows) {
            free(flat_rows), free(hi_rows);
            return -2;
        }
        int any_hi = 0, any_flat = 0;
        for (int r = 0; r < n_rows; ++r) {
            if (idx_row && idx_row[r] != r)
                continue;
            int64_t b = row_seq[r];
            int64_t L = kv_off[b + 1] - kv_off[b];
            if (k_mean && L >= hi_min_len)
                hi_rows[r] = 1, any_hi = 1;
            else
                flat_rows[r] = 1, any_flat = 1;
        }
        (void)n_seq;
        int st = 0;
        if (any_flat) {
            lsa_ref_index_score(dtype, kv_off, n_rows, row_seq, row_pos, q_idx, w, k_idx, HI, dI, k_sink,
                                k_swa, NULL, 0, 1, flat_ws, max_len, flat_rows, n_threads);
            st |= lsa_ref_topk(flat_ws, n_rows, max_len, max_len, NULL, 0, 1, k_sparse, idx, flat_rows,
                               n_threads);
        }
        if (any_hi) {
            st |= lsa_ref_page_recall(dtype, kv_off, sb_off, n_rows, row_seq, row_pos, q_idx, w, k_mean, HI,
                                      dI, P, B, M, page_ws, max_pages, pages_ws, hi_rows, n_threads);
            lsa_ref_index_score(dtype, kv_off, n_rows, row_seq, row_pos, q_idx, w, k_idx, HI, dI, k_sink,
                                k_swa, pages_ws, M, P, comp_ws, M * P, hi_rows, n_threads);
            st |= lsa_ref_topk(comp_ws, n_rows, M * P, M * P, pages_ws, M, P, k_sparse, idx, hi_rows,
                               n_threads);
        }
        free(flat_rows), free(hi_rows);
        if (st)
            return st;
    }
    return lsa_ref_hybrid_attn(dtype, kv_off, n_rows, row_seq, row_pos, q, kv, H, Dqk, Dv, scale, k_sink,
                               k_swa, k_sparse, idx, idx_row, out, lse, n_threads);
}
