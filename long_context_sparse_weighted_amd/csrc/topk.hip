// topk.hip -- exact arg-topK by MSB-first radix select ([paper] §2.2 Eq. 2; SI middle region of
// [review] §2.1; HI stage 2 of [paper] §3.3, which selects Ksparse tokens among recalled pages).
//
// Keys are the order-preserving 32-bit images of the scores (-0 folded onto +0; -inf and NaN are
// not candidates).  The K-th largest key T is fixed digit by digit over three passes (bits 31..21,
// 20..10, 9..0; 2048 bins):
//   hist (per chunk of a row):  LDS histogram of the digit of the keys that still match the prefix
//                               fixed so far, stored as suffix sums (keys in this bin or above);
//                               pass 0 can come straight from the scoring kernel's epilogue;
//   find (one block per row):   sums the chunk suffix histograms, fixes the digit holding the K-th
//                               key, and adds to each chunk's count of keys known to be selected
//                               (those above the fixed digit: one load per chunk); it stops early
//                               when the digit's bin is taken whole;
//   scatter (per chunk):        keys above T are selected; of the keys equal to T, the first
//                               k_rem in position order are (ties go to the lower position); each
//                               chunk writes its picks in position order at its offset in idx, and
//                               the row's tail is padded with -1.
// No global atomics and no fences: on this multi-die part a device-scope fence writes back the
// die's L2, so blocks never synchronise with each other inside a kernel; kernel boundaries order
// the steps.  The result is exact and bitwise deterministic.
#include "lsa_kernels.hpp"

namespace lsa {

constexpr int kBins = kTopkBins;
constexpr int kThreads = 256;
constexpr int kBatch = 16;                      // elements per thread per batch
constexpr int kBatchElems = kThreads * kBatch;  // 4096
constexpr int kMaxChunks = 256;
constexpr int kFindThreads = 1024;

struct TopkState {
    uint32_t prefix;    // fixed top `consumed` bits of T
    uint32_t consumed;  // number of fixed top bits (0, 11, 22 or 32)
    uint32_t k_rem;     // picks still to take among keys whose top bits equal the prefix
    uint32_t done;      // 1: the search has stopped
    uint32_t all;       // 1: at most K candidates, all are picked
    uint32_t ties;      // 1: T fully fixed and only the first k_rem keys equal to T are picked
    uint32_t active;    // row takes part
    uint32_t pad[9];
};
static_assert(sizeof(TopkState) == 64, "state is one 64-byte slot per row");

__host__ __device__ inline int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__host__ __device__ inline int digit_width(int pass) { return pass == 2 ? 10 : 11; }

TopkGeom topk_geometry(int n_rows, int64_t n_cols)
{
    // About two thousand blocks over the whole call, at least one 4096-element batch each.
    int64_t batches = (n_cols + kBatchElems - 1) / kBatchElems;
    if (batches < 1)
        batches = 1;
    int64_t want_chunks = (2048 + n_rows - 1) / n_rows;
    if (want_chunks > kMaxChunks)
        want_chunks = kMaxChunks;
    if (want_chunks > batches)
        want_chunks = batches;
    if (want_chunks < 1)
        want_chunks = 1;
    int64_t per = (batches + want_chunks - 1) / want_chunks;  // batches per chunk
    TopkGeom g;
    g.chunk_elems = per * kBatchElems;
    g.n_chunks = (int)((batches + per - 1) / per);
    return g;
}

TopkWs topk_carve(void *ws, int n_rows, int n_chunks)
{
    char *p = (char *)ws;
    TopkWs t;
    t.state = (TopkState *)p;
    p += align_up(64 * (size_t)n_rows);
    t.hist = (uint32_t *)p;
    p += align_up(sizeof(uint32_t) * kBins * (size_t)n_chunks * n_rows);
    t.chunk_gt = (uint32_t *)p;
    p += align_up(sizeof(uint32_t) * (size_t)n_chunks * n_rows);
    t.chunk_eq = (uint32_t *)p;
    return t;
}

size_t topk_workspace_bytes_geo(int n_rows, int n_chunks)
{
    return align_up(64 * (size_t)n_rows) + align_up(sizeof(uint32_t) * kBins * (size_t)n_chunks * n_rows) +
           2 * align_up(sizeof(uint32_t) * (size_t)n_chunks * n_rows);
}

size_t topk_workspace_bytes(int n_rows, int64_t n_cols)
{
    return topk_workspace_bytes_geo(n_rows, topk_geometry(n_rows, n_cols).n_chunks);
}

// ----------------------------------------------------------------------------------- hist

__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float *__restrict__ scores, int64_t ld,
                                                              int64_t n_cols, const int32_t *pages, int M, int P,
                                                              int pass, TopkGeom geo, TopkWs ws,
                                                              const uint8_t *row_mode, int want)
{
    const int r = blockIdx.y, chunk = blockIdx.x;
    uint32_t prefix = 0, consumed = 0;
    if (pass == 0) {
        if (row_mode && row_mode[r] != want)
            return;
    } else {
        const TopkState *st = ws.state + r;
        if (st->done)
            return;
        prefix = st->prefix;
        consumed = st->consumed;
    }
    __shared__ uint32_t lh[kBins];
    __shared__ uint32_t part[kThreads];
    const int shift = digit_shift(pass);
    const uint32_t dmask = (1u << digit_width(pass)) - 1;
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        lh[i] = 0;
    __syncthreads();
    const float *row = scores + (int64_t)r * ld;
    const int32_t *page_row = pages ? pages + (int64_t)r * M : nullptr;
    const int lane = lane_id();
    const int64_t c_lo = (int64_t)chunk * geo.chunk_elems;
    int64_t c_hi = c_lo + geo.chunk_elems;
    if (c_hi > n_cols)
        c_hi = n_cols;
    for (int64_t c0 = c_lo; c0 < c_hi; c0 += kBatchElems) {
        float sv[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int64_t c = c0 + (int64_t)e * kThreads + threadIdx.x;
            sv[e] = c < c_hi ? row[c] : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int64_t c = c0 + (int64_t)e * kThreads + threadIdx.x;
            bool take = false;
            uint32_t d = 0;
            if (is_candidate(sv[e]) && (!page_row || page_row[(uint32_t)c / (uint32_t)P] >= 0)) {
                const uint32_t key = float_order_key(sv[e]);
                if (consumed == 0 || (key >> (32 - consumed)) == prefix) {
                    take = true;
                    d = (key >> shift) & dmask;
                }
            }
            // Scores of one row crowd into a few bins: lanes that share a digit add it once (one LDS
            // atomic per distinct digit, up to 8 of them); the rest add individually.
            for (int it = 0; it < 8; ++it) {
                const unsigned long long act = __ballot(take);
                if (act == 0)
                    break;
                const int leader = __ffsll((long long)act) - 1;
                const uint32_t dl = (uint32_t)__shfl((int)d, leader, kWave);
                const bool same = take && d == dl;
                const unsigned long long m = __ballot(same);
                if (lane == leader)
                    atomicAdd(&lh[dl], (uint32_t)__popcll(m));
                if (same)
                    take = false;
            }
            if (take)
                atomicAdd(&lh[d], 1u);
        }
    }
    __syncthreads();
    store_suffix_hist(lh, part, ws.hist + ((int64_t)r * geo.n_chunks + chunk) * kBins, kThreads);
}

// ----------------------------------------------------------------------------------- find

__global__ __launch_bounds__(kFindThreads) void topk_find_kernel(int pass, int k, TopkGeom geo, TopkWs ws,
                                                                  const uint8_t *row_mode, int want)
{
    const int r = blockIdx.x;
    TopkState *st = ws.state + r;
    const int t = threadIdx.x;
    uint32_t *gt = ws.chunk_gt + (int64_t)r * geo.n_chunks;
    uint32_t *eq = ws.chunk_eq + (int64_t)r * geo.n_chunks;
    uint32_t k_rem;
    if (pass == 0) {
        const bool active = !row_mode || row_mode[r] == want;
        if (t == 0) {
            st->prefix = 0;
            st->consumed = 0;
            st->k_rem = (uint32_t)k;
            st->done = active ? 0u : 1u;
            st->all = 0;
            st->ties = 0;
            st->active = active ? 1u : 0u;
        }
        for (int c = t; c < geo.n_chunks; c += kFindThreads)
            gt[c] = 0, eq[c] = 0;
        if (!active)
            return;
        k_rem = (uint32_t)k;
    } else {
        if (st->done)
            return;
        k_rem = st->k_rem;
    }
    // Totals of the suffix histograms: group q (256 threads) sums chunks q, q+4, ...; thread (q, u)
    // owns bins [8u, 8u + 8).
    __shared__ uint32_t sfx[4][kBins];
    __shared__ int s_d, s_stop, s_ties;
    const int q = t >> 8, u = t & 255;
    const uint32_t *h = ws.hist + (int64_t)r * geo.n_chunks * kBins;
    {
        uint32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int c = q;
        for (; c + 12 < geo.n_chunks; c += 16) {
            uint4 v[8];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t *hc = h + (int64_t)(c + 4 * x) * kBins + 8 * u;
                v[2 * x] = *reinterpret_cast<const uint4 *>(hc);
                v[2 * x + 1] = *reinterpret_cast<const uint4 *>(hc + 4);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                acc[0] += v[2 * x].x, acc[1] += v[2 * x].y, acc[2] += v[2 * x].z, acc[3] += v[2 * x].w;
                acc[4] += v[2 * x + 1].x, acc[5] += v[2 * x + 1].y, acc[6] += v[2 * x + 1].z,
                    acc[7] += v[2 * x + 1].w;
            }
        }
        for (; c < geo.n_chunks; c += 4) {
            const uint32_t *hc = h + (int64_t)c * kBins + 8 * u;
            const uint4 a = *reinterpret_cast<const uint4 *>(hc), b = *reinterpret_cast<const uint4 *>(hc + 4);
            acc[0] += a.x, acc[1] += a.y, acc[2] += a.z, acc[3] += a.w;
            acc[4] += b.x, acc[5] += b.y, acc[6] += b.z, acc[7] += b.w;
        }
        for (int i = 0; i < 8; ++i)
            sfx[q][8 * u + i] = acc[i];
    }
    __syncthreads();
    if (q == 0)
        for (int i = 0; i < 8; ++i)
            sfx[0][8 * u + i] += sfx[1][8 * u + i] + sfx[2][8 * u + i] + sfx[3][8 * u + i];
    __syncthreads();
    // sfx[0][b] = keys (matching the prefix) in bin b or above; it does not increase with b.
    if (t == 0) {
        const uint32_t total = sfx[0][0];
        if (pass == 0 && total <= k_rem) {
            st->done = 1;  // at most K candidates: every one is picked
            st->all = 1;
            s_d = -1;
        } else {
            int lo = 0, hi = kBins - 1;  // the highest bin whose suffix still reaches k_rem
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sfx[0][mid] >= k_rem)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int d = lo;
            const uint32_t above = d + 1 < kBins ? sfx[0][d + 1] : 0;
            const uint32_t bin = sfx[0][d] - above;
            k_rem -= above;
            const int width = digit_width(pass);
            st->prefix = (st->prefix << width) | (uint32_t)d;
            st->consumed = st->consumed + (uint32_t)width;
            st->k_rem = k_rem;
            const bool whole = bin == k_rem;
            const bool last = pass == 2;
            st->done = (whole || last) ? 1u : 0u;
            st->ties = (last && !whole) ? 1u : 0u;
            s_d = d;
            s_stop = (whole || last) ? 1 : 0;
            s_ties = (last && !whole) ? 1 : 0;
        }
    }
    __syncthreads();
    // Per-chunk counts: keys above the fixed digit are picked; once the search stops, the keys of
    // the fixed bin are either all picked (bin taken whole) or ties of T resolved by position.
    const int d = s_d;
    if (d < 0) {
        for (int c = t; c < geo.n_chunks; c += kFindThreads)
            gt[c] += h[(int64_t)c * kBins];  // every candidate
        return;
    }
    const bool stop = s_stop != 0;
    const bool ties = s_ties != 0;
    for (int c = t; c < geo.n_chunks; c += kFindThreads) {
        const uint32_t *hc = h + (int64_t)c * kBins;
        const uint32_t above = d + 1 < kBins ? hc[d + 1] : 0;
        const uint32_t in_bin = hc[d] - above;
        gt[c] += above;
        if (stop) {
            if (ties)
                eq[c] = in_bin;
            else
                gt[c] += in_bin;
        }
    }
}

// ----------------------------------------------------------------------------------- scatter

__global__ __launch_bounds__(kThreads) void topk_scatter_kernel(const float *__restrict__ scores, int64_t ld,
                                                                 int64_t n_cols, const int32_t *pages, int M, int P,
                                                                 int k, TopkGeom geo, TopkWs ws,
                                                                 int32_t *__restrict__ idx)
{
    const int r = blockIdx.y, chunk = blockIdx.x;
    const TopkState *st = ws.state + r;
    if (!st->active)
        return;
    const uint32_t *gt = ws.chunk_gt + (int64_t)r * geo.n_chunks;
    const uint32_t *eq = ws.chunk_eq + (int64_t)r * geo.n_chunks;
    const bool ties = st->ties != 0;
    const uint32_t k_rem = st->k_rem;
    __shared__ uint32_t s_off, s_total, s_eq_before;
    __shared__ uint32_t cnt_gt[kBatch][kThreads / kWave], cnt_eq[kBatch][kThreads / kWave];
    __shared__ uint32_t off_gt[kBatch][kThreads / kWave], off_eq[kBatch][kThreads / kWave];
    __shared__ uint32_t s_batch_gt, s_batch_eq;
    if (threadIdx.x < kWave) {
        // offset of this chunk = picks of earlier chunks; ties are taken from the left.
        uint32_t before_gt = 0, total_gt = 0, before_eq = 0;
        for (int c = threadIdx.x; c < geo.n_chunks; c += kWave) {
            total_gt += gt[c];
            if (c < chunk) {
                before_gt += gt[c];
                before_eq += eq[c];
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            before_gt += (uint32_t)__shfl_xor((int)before_gt, o, kWave);
            total_gt += (uint32_t)__shfl_xor((int)total_gt, o, kWave);
            before_eq += (uint32_t)__shfl_xor((int)before_eq, o, kWave);
        }
        if (threadIdx.x == 0) {
            const uint32_t taken_eq_before = ties ? (before_eq < k_rem ? before_eq : k_rem) : 0;
            s_off = before_gt + taken_eq_before;
            const uint32_t tot = total_gt + (ties ? k_rem : 0);
            s_total = tot < (uint32_t)k ? tot : (uint32_t)k;
            s_eq_before = before_eq;
        }
    }
    __syncthreads();
    int32_t *out = idx + (int64_t)r * k;
    if (chunk == 0)
        for (int i = (int)s_total + threadIdx.x; i < k; i += kThreads)
            out[i] = -1;
    const uint32_t my_eq = ties ? eq[chunk] : 0;
    if (gt[chunk] == 0 && my_eq == 0)
        return;
    // Ties of this chunk that are picked: the first `take_eq` of them in position order.
    const uint32_t eq_before = s_eq_before;
    const uint32_t room = k_rem > eq_before ? k_rem - eq_before : 0;
    const uint32_t take_eq = ties ? (my_eq < room ? my_eq : room) : 0;
    const uint32_t prefix = st->prefix, consumed = st->consumed;
    const bool all = st->all != 0;
    const float *row = scores + (int64_t)r * ld;
    const int32_t *page_row = pages ? pages + (int64_t)r * M : nullptr;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t c_lo = (int64_t)chunk * geo.chunk_elems;
    int64_t c_hi = c_lo + geo.chunk_elems;
    if (c_hi > n_cols)
        c_hi = n_cols;
    // gt: picked for sure (above T, or in a bin taken whole); eq: equal to T when ties are split.
    auto classify = [&](float s, int64_t c, bool &g, bool &e) {
        g = e = false;
        if (!is_candidate(s) || (page_row && page_row[(uint32_t)c / (uint32_t)P] < 0))
            return;
        if (all) {
            g = true;
            return;
        }
        const uint32_t top = float_order_key(s) >> (32 - consumed);
        if (ties) {
            g = top > prefix;
            e = top == prefix;
        } else {
            g = top >= prefix;
        }
    };
    uint32_t run_gt = 0, run_eq = 0;  // picks / ties of this chunk before the current batch
    const unsigned long long below = (1ull << lane) - 1;
    for (int64_t c0 = c_lo; c0 < c_hi; c0 += kBatchElems) {
        float sv[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int64_t c = c0 + (int64_t)e * kThreads + threadIdx.x;
            sv[e] = c < c_hi ? row[c] : -INFINITY;
        }
        // Position order inside a batch is (step e, wave, lane): count per (e, wave) first ...
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int64_t c = c0 + (int64_t)e * kThreads + threadIdx.x;
            bool g, q;
            classify(sv[e], c, g, q);
            const unsigned long long mg = __ballot(g), mq = __ballot(q);
            if (lane == 0) {
                cnt_gt[e][wave] = (uint32_t)__popcll(mg);
                cnt_eq[e][wave] = (uint32_t)__popcll(mq);
            }
        }
        __syncthreads();
        if (threadIdx.x < kWave) {
            // the 64 (step, wave) counts in position order, scanned by one wave
            static_assert(kBatch * (kThreads / kWave) == kWave, "one lane per (step, wave)");
            const int e = threadIdx.x >> 2, w = threadIdx.x & 3;
            const uint32_t a = cnt_gt[e][w], b = cnt_eq[e][w];
            uint32_t ia = a, ib = b;
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t ya = (uint32_t)__shfl_up((int)ia, o, kWave);
                const uint32_t yb = (uint32_t)__shfl_up((int)ib, o, kWave);
                if (threadIdx.x >= o)
                    ia += ya, ib += yb;
            }
            off_gt[e][w] = ia - a;
            off_eq[e][w] = ib - b;
            if (threadIdx.x == kWave - 1)
                s_batch_gt = ia, s_batch_eq = ib;
        }
        __syncthreads();
        // ... then write: a tie is picked while its rank among the chunk's ties is below take_eq.
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int64_t c = c0 + (int64_t)e * kThreads + threadIdx.x;
            bool g, q;
            classify(sv[e], c, g, q);
            const unsigned long long mg = __ballot(g), mq = __ballot(q);
            const uint32_t gt_before = run_gt + off_gt[e][wave] + (uint32_t)__popcll(mg & below);
            const uint32_t eq_rank = run_eq + off_eq[e][wave] + (uint32_t)__popcll(mq & below);
            const bool pick = g || (q && eq_rank < take_eq);
            if (pick) {
                const uint32_t eq_picked_before = eq_rank < take_eq ? eq_rank : take_eq;
                const uint32_t slot = s_off + gt_before + eq_picked_before;
                const int64_t pos =
                    page_row ? (int64_t)page_row[(uint32_t)c / (uint32_t)P] * P + (uint32_t)c % (uint32_t)P : c;
                if (slot < (uint32_t)k)
                    out[slot] = (int32_t)pos;
            }
        }
        run_gt += s_batch_gt;
        run_eq += s_batch_eq;
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------------- host

hipError_t launch_topk_geo(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M,
                           int P, int k, int32_t *idx, void *ws_ptr, TopkGeom geo, bool pass0_done, RowGate gate,
                           hipStream_t stream)
{
    if (n_rows == 0)
        return hipSuccess;
    TopkWs ws = topk_carve(ws_ptr, n_rows, geo.n_chunks);
    const dim3 grid(geo.n_chunks, n_rows);
    const int64_t nc = n_cols > 0 ? n_cols : 0;
    for (int p = 0; p < 3; ++p) {
        if (p > 0 || !pass0_done)
            hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, scores, ld, nc, pages, M, P, p, geo,
                               ws, gate.row_mode, gate.want);
        hipLaunchKernelGGL(topk_find_kernel, dim3(n_rows), dim3(kFindThreads), 0, stream, p, k, geo, ws,
                           gate.row_mode, gate.want);
    }
    hipLaunchKernelGGL(topk_scatter_kernel, grid, dim3(kThreads), 0, stream, scores, ld, nc, pages, M, P, k, geo, ws,
                       idx);
    return hipGetLastError();
}

hipError_t launch_topk(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M, int P,
                       int k, int32_t *idx, void *ws_ptr, RowGate gate, hipStream_t stream)
{
    const TopkGeom geo = topk_geometry(n_rows, n_cols > 0 ? n_cols : 1);
    return launch_topk_geo(n_rows, scores, ld, n_cols, pages, M, P, k, idx, ws_ptr, geo, false, gate, stream);
}

}  // namespace lsa
