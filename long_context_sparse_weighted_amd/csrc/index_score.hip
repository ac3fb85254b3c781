// index_score.hip -- Lightning-Indexer scoring on gfx950.
//
// I(t, s) = sum_j w(t, j) * ReLU(q(t, j) . k(s))        ([paper] §2.2 Eq. 1, MQA-shared key)
// evaluated only on the SI middle region mid(t) ([paper] §3.1 "Design choices" (b); [review] §2.1),
// on the tokens of recalled pages (HI stage 2, [paper] §3.3), or on cached sub-block means summed
// per page (HI stage 1, [paper] §3.3 "Block-level coarse filtering").
//
// bf16 path (64 heads x 128 dims): one wave computes a [64 heads x 16 keys] tile with
// v_mfma_f32_16x16x32_bf16 (4 head tiles x 4 depth steps).  The query's 64x128 block stays in
// VGPRs for the whole wave; keys stream from HBM, 16 keys (4 KB) per tile.  The epilogue applies ReLU and the head weights in
// registers and reduces the 64 heads across the 4 lane groups with two xor shuffles; nothing but the
// fp32 score (4 B per key) is written.  Three tiles rotate through registers, so two 4 KB loads
// per wave are in flight while the third tile is multiplied.  Step ks of the MFMA reads bytes
// [64ks, 64ks + 64) of each of the 16 key rows (lane group g takes the 16 bytes at 64ks + 16g), so
// each load instruction covers whole half-lines; two steps complete a 128-byte line while it is
// still in L2.  Keys are read with ordinary (cached) loads: a streaming hint would drop the line
// before its second half is read.
//
// fp32 path: one thread per key with the key row in VGPRs and q / w in LDS (small configs).
#include "lsa_kernels.hpp"

namespace lsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { kModeFlat = 0, kModePaged = 1, kModePageMean = 2 };

// Per-row view of which key a column stands for.
struct ColMap {
    int64_t base;       // first key row of the sequence (k_idx) or of its means (k_mean)
    int64_t lo, hi;     // FLAT/PAGED: valid positions [lo, hi) = mid(t) cut at L
    int64_t nsb;        // PAGEMEAN: sub-blocks of the sequence
    int64_t last_page;  // PAGEMEAN: pages p <= last_page are causal and exist
    int G;              // PAGEMEAN: sub-blocks per page
    int P;              // PAGED: page size
    const int32_t *page_row;
    int M;
};

template <int MODE>
__device__ inline ColMap make_colmap(const RowInfo &ri, const SiRanges &g, const int64_t *sb_off, const int32_t *pages,
                                     int r, int M, int P, int B)
{
    ColMap m;
    m.base = ri.base;
    m.lo = g.mid_lo;
    m.hi = g.mid_hi < ri.L ? g.mid_hi : ri.L;
    m.nsb = 0;
    m.last_page = -1;
    m.G = 1;
    m.P = P;
    m.page_row = pages ? pages + (int64_t)r * M : nullptr;
    m.M = M;
    if (MODE == kModePageMean) {
        if (ri.valid) {
            m.base = sb_off[ri.seq];
            m.nsb = sb_off[ri.seq + 1] - m.base;
            int64_t n_pages = (ri.L + P - 1) / P;
            int64_t tp = ri.t / P;
            m.last_page = tp < n_pages - 1 ? tp : n_pages - 1;
        }
        m.G = P / B;
    }
    return m;
}

// Key row of column c (or -1 when the column holds no score).
template <int MODE>
__device__ inline int64_t col_key(const ColMap &m, int64_t c)
{
    if (MODE == kModeFlat) {
        return (c >= m.lo && c < m.hi) ? m.base + c : -1;
    } else if (MODE == kModePaged) {
        int64_t slot = c / m.P;
        if (slot >= m.M)
            return -1;
        int64_t pg = m.page_row[slot];
        if (pg < 0)
            return -1;
        int64_t s = pg * m.P + c % m.P;
        return (s >= m.lo && s < m.hi) ? m.base + s : -1;
    } else {
        return (c < m.nsb && c / m.G <= m.last_page) ? m.base + c : -1;
    }
}

// ------------------------------------------------------------------------------------------
// bf16 matrix-core kernel: 64 indexer heads x 128 dims.

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kTile = 16;          // keys per MFMA tile
constexpr int kWavesPerBlock = 4;

template <int MODE>
__global__ __launch_bounds__(256) void score_mfma_kernel(RowsDev rows, const uint16_t *__restrict__ q_idx,
                                                          const float *__restrict__ w,
                                                          const uint16_t *__restrict__ keys, int k_sink, int k_swa,
                                                          const int64_t *sb_off, const int32_t *pages, int M, int P,
                                                          int B, float *__restrict__ scores, int64_t ld,
                                                          int64_t n_cols, int64_t cols_per_block,
                                                          const uint8_t *row_mode, int want, uint32_t *topk_hist)
{
    const int r = blockIdx.y;
    if (row_mode && row_mode[r] != want)
        return;
    // Optional fused first pass of the top-K that follows: a histogram of the top 11 bits of the
    // order-preserving image of every score this block writes (one chunk = this block's columns).
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t part[256];
    const bool fuse_hist = MODE != kModePageMean && topk_hist != nullptr;
    if (fuse_hist) {
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x)
            lh[i] = 0;
        __syncthreads();
    }
    const RowInfo ri = row_info(rows, r);
    const SiRanges si = si_ranges(ri, k_sink, k_swa);
    const ColMap cm = make_colmap<MODE>(ri, si, sb_off, pages, r, M, P, B);

    const int lane = lane_id();
    const int n = lane & 15;  // key column within the tile / head row within an MFMA tile
    const int g = lane >> 4;  // lane group: depth 32ks + 8g .. +8 of step ks; heads 4g..4g+3 of each tile
    const int wave = threadIdx.x >> 6;

    const int64_t c_begin = (int64_t)blockIdx.x * cols_per_block;
    int64_t c_end = c_begin + cols_per_block;
    if (c_end > n_cols)
        c_end = n_cols;
    float *out = scores + (int64_t)r * ld;

    // A operands: q rows of this query, head mt*16 + n, depth 32ks + 8g .. +8.
    u32x4 qa[4][4];
    const uint16_t *qrow = q_idx + (int64_t)r * kHeads * kDim;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qrow + (mt * 16 + n) * kDim + g * 8);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qa[mt][ks] = src[4 * ks];
    }
    // Head weights of the 16 heads whose dot products this lane ends up holding.
    float wv[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(w + (int64_t)r * kHeads + mt * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wv[mt][i] = v[i];
    }

    const int64_t first_tile = c_begin / kTile + wave;
    const int64_t end_tile = (c_end + kTile - 1) / kTile;

    // A row with nothing to score writes -inf over its columns and issues no loads.
    const bool row_has_keys = MODE == kModePageMean ? cm.nsb > 0 : cm.lo < cm.hi;
    if (!row_has_keys) {
        if (fuse_hist)
            store_suffix_hist(lh, part, topk_hist + ((int64_t)r * gridDim.x + blockIdx.x) * kTopkBins, 256);
        if (MODE == kModePageMean) {
            for (int64_t p = c_begin / cm.G + threadIdx.x; p < (c_end + cm.G - 1) / cm.G && p < ld; p += blockDim.x)
                out[p] = -INFINITY;
        } else {
            for (int64_t c = c_begin + threadIdx.x; c < c_end; c += blockDim.x)
                out[c] = -INFINITY;
        }
        return;
    }
    // Columns without a score still load a row of the sequence (its first scored key), so every
    // load is unconditional and the loads of later tiles stay in flight across iterations.
    const int64_t safe_key = MODE == kModePageMean ? cm.base : cm.base + cm.lo;
    auto load_tile = [&](int64_t tile, u32x4 (&b)[4], int64_t &key) {
        key = col_key<MODE>(cm, tile * kTile + n);
        const int64_t row_k = key >= 0 ? key : safe_key;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(keys + row_k * kDim + g * 8);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            b[ks] = src[4 * ks];
    };

    // One tile: MFMAs, ReLU + head weights, reduction over the 4 lane groups, store.
    auto compute = [&](int64_t tile, const u32x4 (&b)[4], int64_t key) {
        const bool any = __ballot(key >= 0) != 0;  // wave-uniform
        float v = 0.0f;
        if (any) {
            f32x4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 bb = __builtin_bit_cast(bf16x8, b[ks]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[mt][ks]), bb,
                                                                      acc[mt], 0, 0, 0);
            }
            // acc[mt][i] = q(head mt*16 + 4g + i) . k(column n)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v += wv[mt][i] * fmaxf(acc[mt][i], 0.0f);
            v += __shfl_xor(v, 16, kWave);
            v += __shfl_xor(v, 32, kWave);
        }
        const int64_t c = tile * kTile + n;
        if (MODE == kModePageMean) {
            // Sum the G sub-blocks of each page (they are G consecutive columns of this tile); a
            // sub-block that does not exist adds nothing.
            if (key < 0)
                v = 0.0f;
            for (int o = 1; o < cm.G; o <<= 1)
                v += __shfl_xor(v, o, kWave);
            // (every lane group holds the same sums; all of them store, without branching)
            const int64_t p = c / cm.G;
            if ((n % cm.G) == 0 && p < ld)
                out[p] = (p <= cm.last_page) ? v : -INFINITY;
        } else if (c < c_end) {
            out[c] = key >= 0 ? v : -INFINITY;
            if (fuse_hist && g == 0 && key >= 0)
                atomicAdd(&lh[float_order_key(v) >> 21], 1u);
        }
    };

    // Three register buffers: two tiles are in flight while the third is multiplied.
    constexpr int64_t W = kWavesPerBlock;
    u32x4 b0[4], b1[4], b2[4];
    int64_t k0 = -1, k1 = -1, k2 = -1;
    int64_t tile = first_tile;
    load_tile(tile, b0, k0);
    load_tile(tile + W, b1, k1);
    for (; tile < end_tile; tile += 3 * W) {
        load_tile(tile + 2 * W, b2, k2);
        compute(tile, b0, k0);
        load_tile(tile + 3 * W, b0, k0);
        if (tile + W < end_tile)
            compute(tile + W, b1, k1);
        load_tile(tile + 4 * W, b1, k1);
        if (tile + 2 * W < end_tile)
            compute(tile + 2 * W, b2, k2);
    }
    if (fuse_hist) {
        __syncthreads();
        store_suffix_hist(lh, part, topk_hist + ((int64_t)r * gridDim.x + blockIdx.x) * kTopkBins, 256);
    }
}

// ------------------------------------------------------------------------------------------
// fp32 VALU kernel (any n_heads <= 64, head_dim in {64, 128}); one thread per column.

template <int DI, int MODE>
__global__ __launch_bounds__(256) void score_valu_kernel(RowsDev rows, const float *__restrict__ q_idx,
                                                          const float *__restrict__ w, const float *__restrict__ keys,
                                                          int n_heads, int k_sink, int k_swa, const int64_t *sb_off,
                                                          const int32_t *pages, int M, int P, int B,
                                                          float *__restrict__ scores, int64_t ld, int64_t n_cols,
                                                          const uint8_t *row_mode, int want)
{
    const int r = blockIdx.y;
    if (row_mode && row_mode[r] != want)
        return;
    __shared__ float qs[kHeads * DI];
    __shared__ float ws[kHeads];
    for (int i = threadIdx.x; i < n_heads * DI; i += blockDim.x)
        qs[i] = q_idx[(int64_t)r * n_heads * DI + i];
    for (int i = threadIdx.x; i < n_heads; i += blockDim.x)
        ws[i] = w[(int64_t)r * n_heads + i];
    __syncthreads();
    const RowInfo ri = row_info(rows, r);
    const SiRanges si = si_ranges(ri, k_sink, k_swa);
    const ColMap cm = make_colmap<MODE>(ri, si, sb_off, pages, r, M, P, B);
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n_cols)
        return;
    float *out = scores + (int64_t)r * ld;

    auto key_score = [&](int64_t key) {
        float kr[DI];
        const f32x4 *src = reinterpret_cast<const f32x4 *>(keys + key * DI);
#pragma unroll
        for (int d4 = 0; d4 < DI / 4; ++d4) {
            f32x4 v = src[d4];
            kr[4 * d4 + 0] = v[0], kr[4 * d4 + 1] = v[1], kr[4 * d4 + 2] = v[2], kr[4 * d4 + 3] = v[3];
        }
        float acc = 0.0f;
        for (int j = 0; j < n_heads; ++j) {
            float dot = 0.0f;
#pragma unroll
            for (int d = 0; d < DI; ++d)
                dot = fmaf(qs[j * DI + d], kr[d], dot);
            acc = fmaf(ws[j], fmaxf(dot, 0.0f), acc);
        }
        return acc;
    };

    if (MODE == kModePageMean) {
        // column c is page c: sum over its G sub-blocks
        if (c >= ld)
            return;
        if (c > cm.last_page) {
            out[c] = -INFINITY;
            return;
        }
        float acc = 0.0f;
        for (int i = 0; i < cm.G; ++i) {
            int64_t key = col_key<MODE>(cm, c * cm.G + i);
            if (key >= 0)
                acc += key_score(key);
        }
        out[c] = acc;
    } else {
        int64_t key = col_key<MODE>(cm, c);
        out[c] = key >= 0 ? key_score(key) : -INFINITY;
    }
}

// ------------------------------------------------------------------------------------------ host

bool index_score_supported(int dtype, int n_heads, int head_dim)
{
    if (dtype == 1)
        return n_heads == kHeads && head_dim == kDim;
    return n_heads >= 1 && n_heads <= kHeads && (head_dim == 64 || head_dim == 128);
}

// Columns per block for the MFMA kernel: enough blocks to cover the chip a few times over.
static int64_t pick_cols_per_block(int64_t n_rows, int64_t n_cols)
{
    int64_t total = n_rows * n_cols;
    int64_t cpb = total / 2048;
    cpb = (cpb + 63) / 64 * 64;
    if (cpb < 256)
        cpb = 256;
    if (cpb > 16384)
        cpb = 16384;
    return cpb;
}

TopkGeom score_geometry(int dtype, int n_rows, int64_t n_cols)
{
    if (dtype != 1)
        return topk_geometry(n_rows, n_cols);
    TopkGeom g;
    g.chunk_elems = pick_cols_per_block(n_rows, n_cols);
    g.n_chunks = (int)((n_cols + g.chunk_elems - 1) / g.chunk_elems);
    return g;
}

template <int MODE>
static hipError_t launch_mode(int dtype, const RowsDev &rows, const void *q_idx, const float *w, const void *keys,
                              int n_heads, int head_dim, int k_sink, int k_swa, const int64_t *sb_off,
                              const int32_t *pages, int M, int P, int B, float *scores, int64_t ld, int64_t n_cols,
                              RowGate gate, hipStream_t stream, uint32_t *topk_hist = nullptr)
{
    if (rows.n_rows == 0 || n_cols == 0)
        return hipSuccess;
    if (dtype == 1) {
        const TopkGeom geo = score_geometry(dtype, rows.n_rows, n_cols);
        dim3 grid((unsigned)geo.n_chunks, (unsigned)rows.n_rows);
        hipLaunchKernelGGL(score_mfma_kernel<MODE>, grid, dim3(256), 0, stream, rows, (const uint16_t *)q_idx, w,
                           (const uint16_t *)keys, k_sink, k_swa, sb_off, pages, M, P, B, scores, ld, n_cols,
                           geo.chunk_elems, gate.row_mode, gate.want, topk_hist);
    } else {
        int64_t threads_cols = MODE == kModePageMean ? ld : n_cols;
        dim3 grid((unsigned)((threads_cols + 255) / 256), (unsigned)rows.n_rows);
        if (head_dim == 64)
            hipLaunchKernelGGL((score_valu_kernel<64, MODE>), grid, dim3(256), 0, stream, rows, (const float *)q_idx, w,
                               (const float *)keys, n_heads, k_sink, k_swa, sb_off, pages, M, P, B, scores, ld,
                               threads_cols, gate.row_mode, gate.want);
        else
            hipLaunchKernelGGL((score_valu_kernel<128, MODE>), grid, dim3(256), 0, stream, rows, (const float *)q_idx,
                               w, (const float *)keys, n_heads, k_sink, k_swa, sb_off, pages, M, P, B, scores, ld,
                               threads_cols, gate.row_mode, gate.want);
    }
    return hipGetLastError();
}

hipError_t launch_index_score(int dtype, const RowsDev &rows, int64_t max_kv_len, const void *q_idx, const float *w,
                              const void *k_idx, int n_heads, int head_dim, int k_sink, int k_swa,
                              const int32_t *pages, int M, int P, float *scores, int64_t ld, RowGate gate,
                              hipStream_t stream, uint32_t *topk_hist)
{
    (void)max_kv_len;
    if (pages)
        return launch_mode<kModePaged>(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, k_sink, k_swa, nullptr, pages,
                                       M, P, 1, scores, ld, ld, gate, stream, topk_hist);
    return launch_mode<kModeFlat>(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, k_sink, k_swa, nullptr, nullptr,
                                  0, 1, 1, scores, ld, ld, gate, stream, topk_hist);
}

hipError_t launch_page_scores(int dtype, const RowsDev &rows, int64_t max_kv_len, const int64_t *sb_off,
                              const void *q_idx, const float *w, const void *k_mean, int n_heads, int head_dim,
                              int P, int B, float *page_scores, int64_t ld_ps, RowGate gate, hipStream_t stream)
{
    (void)max_kv_len;
    const int G = P / B;
    // Sub-block columns: ld_ps pages x G sub-blocks, so every page column is produced by one tile.
    return launch_mode<kModePageMean>(dtype, rows, q_idx, w, k_mean, n_heads, head_dim, 0, 0, sb_off, nullptr, 0, P,
                                      B, page_scores, ld_ps, ld_ps * G, gate, stream);
}

}  // namespace lsa
