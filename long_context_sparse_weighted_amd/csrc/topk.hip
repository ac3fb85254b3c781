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

size_t topk2_workspace_bytes(int n_rows, int64_t n_cols, int k);
bool topk_two_level(int k);

size_t topk_workspace_bytes(int n_rows, int64_t n_cols, int k)
{
    if (topk_two_level(k))
        return topk2_workspace_bytes(n_rows, n_cols > 0 ? n_cols : 1, k);
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

// ----------------------------------------------------------------------------------- two-level
//
// For k <= kMaxLocalK the selection runs in two levels instead of the passes above.  A block holds a
// segment of up to 64 * NT keys in registers (thread t holds positions 64 t .. 64 t + 63 of the
// segment) and selects its best k under (key desc, position asc) by the same radix steps, on LDS
// histograms.  Level 1 cuts each row into segments of kSeg scores and writes every segment's picks
// (candidates: key and position, in position order, padded with key 0) -- the row's top k is among
// them, since an element with fewer than k better elements in the row has fewer than k better
// elements in its segment.  Further levels do the same on the candidate lists (whose order is
// still position order) until one segment per row remains, whose picks are the result.  Scores
// are read once.

constexpr int kVpt = 64;                        // keys per thread
constexpr int kSegThreads = 256;
constexpr int kSeg = kVpt * kSegThreads;        // 16384
constexpr int kMaxLocalK = 4096;

// Exclusive prefix sums over threads (in thread order) of two counters, and their totals.
// scratch: 2 * NT / 64 words of LDS.
template <int NT>
__device__ __attribute__((always_inline)) inline void block_scan2(uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb, uint32_t &ta, uint32_t &tb,
                                   uint32_t *scratch)
{
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    uint32_t ia = a, ib = b;
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t ya = (uint32_t)__shfl_up((int)ia, o, kWave), yb = (uint32_t)__shfl_up((int)ib, o, kWave);
        if (lane >= o)
            ia += ya, ib += yb;
    }
    if (lane == kWave - 1)
        scratch[w] = ia, scratch[NW + w] = ib;
    __syncthreads();
    uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t xa = scratch[i], xb = scratch[NW + i];
        if (i < w)
            pa += xa, pb += xb;
        sa += xa, sb += xb;
    }
    ea = pa + ia - a, eb = pb + ib - b, ta = sa, tb = sb;
    __syncthreads();
}

struct Selection {
    uint32_t prefix;    // fixed top `consumed` bits of the threshold
    int consumed;
    uint32_t k_rem;     // keys equal to the threshold that are picked (first in position order)
    bool whole;         // keys whose top bits equal the prefix are all picked
    bool all;           // every candidate is picked
};

// Radix select of the block's best k among the non-zero keys (0 = not a candidate).  The digit
// histograms live in LDS as kCopies interleaved copies (bin b, copy c at hist[kCopies b + c]; lane l
// adds to copy l % kCopies): keys of one row crowd into a few bins, and the copies spread the
// atomics on such a bin over consecutive banks.  Keys that do not take part add to a per-lane
// dummy word instead (no branch per key).
constexpr int kCopies = 2;
constexpr int kHistWords = kBins * kCopies + kWave;  // + one dummy word per lane
constexpr int kStageWords = 2 * (kMaxLocalK + kWave);
constexpr int kLdsWords = kHistWords > kStageWords ? kHistWords : kStageWords;

template <int NT>
__device__ __attribute__((always_inline)) Selection block_select(const uint32_t (&key)[kVpt], uint32_t k,
                                                                 uint32_t *hist, uint32_t *scratch, int *s_d,
                                                                 uint32_t *s_above, uint32_t *s_bin)
{
    Selection sel{0u, 0, k, false, false};
    uint32_t cnt = 0;
#pragma unroll
    for (int m = 0; m < kVpt; ++m)
        cnt += key[m] != 0 ? 1u : 0u;
    uint32_t e0, e1, total, t1;
    block_scan2<NT>(cnt, 0, e0, e1, total, t1, scratch);
    if (total <= k) {
        sel.all = true;
        return sel;
    }
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t copy = lane % kCopies, dummy = kBins * kCopies + lane;
    constexpr int kPer = kBins / NT;  // bins owned by a thread in the suffix scan
    // Cleared once here; afterwards every pass clears the words it has read.
    for (int i = threadIdx.x; i < kBins * kCopies / 4; i += NT)
        reinterpret_cast<uint4 *>(hist)[i] = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = digit_shift(pass);
        const uint32_t dmask = (1u << digit_width(pass)) - 1;
        // keys whose top `consumed` bits equal the prefix: (x & pmask) == pval (uniform scalars)
        const uint32_t pmask = sel.consumed == 0 ? 0u : ~0u << (32 - sel.consumed);
        const uint32_t pval = sel.consumed == 0 ? 0u : sel.prefix << (32 - sel.consumed);
        // (Key 0, not a candidate, falls in pass-0 bin 0, below every candidate key: a digit
        // below 3 is never selected while there are more than k candidates.)
#pragma unroll
        for (int m = 0; m < kVpt; ++m) {
            const uint32_t x = key[m];
            const bool take = (x & pmask) == pval;
            atomicAdd(&hist[take ? kCopies * ((x >> shift) & dmask) + copy : dummy], 1u);
        }
        __syncthreads();
        // Suffix sums (keys in bin b or above): thread t owns bins [kPer t, kPer t + kPer).
        uint32_t hb[kPer];
        uint32_t own = 0;
        constexpr int kWords = kPer * kCopies;  // this thread's words, read (and cleared) 16 bytes at a time
        static_assert(kWords % 4 == 0, "whole 16-byte words");
        uint32_t wv[kWords];
        uint4 *hw = reinterpret_cast<uint4 *>(hist + kWords * threadIdx.x);
#pragma unroll
        for (int q = 0; q < kWords / 4; ++q) {
            const uint4 x = hw[q];
            wv[4 * q] = x.x, wv[4 * q + 1] = x.y, wv[4 * q + 2] = x.z, wv[4 * q + 3] = x.w;
            hw[q] = uint4{0u, 0u, 0u, 0u};  // ready for the next pass
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            uint32_t v = 0;
#pragma unroll
            for (int c = 0; c < kCopies; ++c)
                v += wv[kCopies * i + c];
            hb[i] = v;
            own += v;
        }
        uint32_t before, unused, sum_all, unused2;
        block_scan2<NT>(own, 0, before, unused, sum_all, unused2, scratch);
        uint32_t run = sum_all - before - own;  // keys in bins above this thread's
#pragma unroll
        for (int i = kPer - 1; i >= 0; --i) {
            if (run < sel.k_rem && run + hb[i] >= sel.k_rem) {  // the bin holding the k_rem-th key
                *s_d = kPer * threadIdx.x + i;
                *s_above = run;
                *s_bin = hb[i];
            }
            run += hb[i];
        }
        __syncthreads();
        const int d = *s_d;
        const uint32_t above = *s_above, bin = *s_bin;
        __syncthreads();
        sel.k_rem -= above;
        sel.prefix = (sel.prefix << digit_width(pass)) | (uint32_t)d;
        sel.consumed += digit_width(pass);
        if (bin == sel.k_rem) {
            sel.whole = true;
            break;
        }
    }
    return sel;
}

// Writes the picks of a selection, in position order, to stage_key / stage_li (key and index in
// the segment) at slots 0 .. n - 1 and returns n; keys not picked go to per-lane dummy slots
// stage[kMaxLocalK + lane].
template <int NT>
__device__ __attribute__((always_inline)) uint32_t block_emit(const uint32_t (&key)[kVpt], const Selection &sel,
                                                              uint32_t *scratch, uint32_t *stage_key,
                                                              uint32_t *stage_li, uint32_t first_li)
{
    // Thresholds on the whole key (uniform): picked for sure when x >= t_gt; a tie when x == t_eq.
    //   all: every candidate;  whole: keys with top bits >= prefix;  otherwise T is exact
    //   (32 bits fixed): x > T picked, x == T a tie.
    //   (0xffffffff is a NaN pattern, mapped to key 0: no key equals it.)
    uint32_t t_gt, t_eq = 0xffffffffu;
    if (sel.all) {
        t_gt = 1u;
    } else if (sel.whole) {
        t_gt = sel.prefix << (32 - sel.consumed);
    } else {
        t_gt = sel.prefix + 1u, t_eq = sel.prefix;  // consumed == 32: prefix is T
    }
    // Flags of this thread's keys as bit masks (bit m: key m).
    uint64_t gbits = 0, ebits = 0;
#pragma unroll
    for (int m = 0; m < kVpt; ++m) {
        gbits |= (uint64_t)(key[m] >= t_gt ? 1u : 0u) << m;
        ebits |= (uint64_t)(key[m] == t_eq ? 1u : 0u) << m;
    }
    const uint32_t cg = (uint32_t)__popcll(gbits), ce = (uint32_t)__popcll(ebits);
    uint32_t bg, be, tg, te;
    block_scan2<NT>(cg, ce, bg, be, tg, te, scratch);
    const uint32_t dummy = kMaxLocalK + (uint32_t)lane_id();
#pragma unroll
    for (int m = 0; m < kVpt; ++m) {
        const bool g = (gbits >> m) & 1u, e = (ebits >> m) & 1u;
        const bool pick = g || (e && be < sel.k_rem);
        const uint32_t slot = pick ? bg + (be < sel.k_rem ? be : sel.k_rem) : dummy;
        stage_key[slot] = key[m];
        stage_li[slot] = first_li + m;
        bg += g ? 1u : 0u;
        be += e ? 1u : 0u;
    }
    return tg + (te < sel.k_rem ? te : sel.k_rem);
}

// One level.  SRC_SCORES: segment `seg` of row r is columns [seg * 64 NT, ...) of the scores (page
// mapped when pages is given; P is a multiple of 16, so 16 aligned columns share a page);
// otherwise candidates [seg * 64 NT, ...) of row r's list of n_in.  FINAL: the picks (positions)
// go to idx[r][0 .. k), padded with -1; otherwise to the next list at [seg * k, seg * k + k),
// padded with key 0.
template <int NT, bool SRC_SCORES, bool FINAL>
__global__ __launch_bounds__(NT) void topk_level_kernel(const float *__restrict__ scores, int64_t ld, int64_t n_in,
                                                         const int32_t *__restrict__ pages, int M, int P,
                                                         const uint32_t *__restrict__ in_key,
                                                         const int32_t *__restrict__ in_pos, int64_t in_ld, int k,
                                                         uint32_t *__restrict__ out_key, int32_t *__restrict__ out_pos,
                                                         int64_t out_ld, int32_t *__restrict__ idx,
                                                         const uint8_t *row_mode, int want)
{
    const int seg = blockIdx.x, r = blockIdx.y;
    if (row_mode && row_mode[r] != want)
        return;
    // LDS: the histograms, reused afterwards as the staging area of the picks.
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
    __shared__ uint32_t scratch[2 * NT / kWave];
    __shared__ int s_d;
    __shared__ uint32_t s_above, s_bin;
    const int64_t seg_base = (int64_t)seg * (kVpt * NT);
    const int64_t base = seg_base + (int64_t)kVpt * threadIdx.x;  // this thread's first element
    const int32_t *page_row = pages ? pages + (int64_t)r * M : nullptr;
    uint32_t key[kVpt];
    if constexpr (SRC_SCORES) {
        const float *row = scores + (int64_t)r * ld;
        if (base + kVpt <= n_in && (ld & 3) == 0 && ((uintptr_t)scores & 15) == 0) {
            const float4 *src = reinterpret_cast<const float4 *>(row + base);
#pragma unroll
            for (int q = 0; q < kVpt / 4; ++q) {
                const float4 v = src[q];
                key[4 * q] = is_candidate(v.x) ? float_order_key(v.x) : 0u;
                key[4 * q + 1] = is_candidate(v.y) ? float_order_key(v.y) : 0u;
                key[4 * q + 2] = is_candidate(v.z) ? float_order_key(v.z) : 0u;
                key[4 * q + 3] = is_candidate(v.w) ? float_order_key(v.w) : 0u;
            }
        } else {
#pragma unroll
            for (int m = 0; m < kVpt; ++m) {
                const int64_t c = base + m;
                const float v = c < n_in ? row[c] : -INFINITY;
                key[m] = is_candidate(v) ? float_order_key(v) : 0u;
            }
        }
        if (page_row) {
#pragma unroll
            for (int q = 0; q < kVpt / 16; ++q) {
                const int64_t c = base + 16 * q;
                const bool ok = c < n_in && page_row[(uint32_t)c / (uint32_t)P] >= 0;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    key[16 * q + i] = ok ? key[16 * q + i] : 0u;
            }
        }
    } else {
        const uint32_t *src = in_key + (int64_t)r * in_ld;
        if (base + kVpt <= n_in) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(src + base);
#pragma unroll
            for (int q = 0; q < kVpt / 4; ++q) {
                const uint4 v = s4[q];
                key[4 * q] = v.x, key[4 * q + 1] = v.y, key[4 * q + 2] = v.z, key[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < kVpt; ++m)
                key[m] = base + m < n_in ? src[base + m] : 0u;
        }
    }
    const Selection sel = block_select<NT>(key, (uint32_t)k, lds, scratch, &s_d, &s_above, &s_bin);
    uint32_t *stage_key = lds, *stage_li = lds + kMaxLocalK + kWave;
    __syncthreads();  // the histograms are no longer read
    const uint32_t n_sel = block_emit<NT>(key, sel, scratch, stage_key, stage_li, (uint32_t)(kVpt * threadIdx.x));
    __syncthreads();
    // Copy-out in slot order (coalesced), with positions computed for the picks only.
    for (int i = threadIdx.x; i < k; i += NT) {
        int32_t pos = -1;
        uint32_t kv = 0;
        const int64_t c = seg_base + stage_li[i];
        if ((uint32_t)i < n_sel && c < n_in) {  // (a pick is always below n_in: keys past it are 0)
            kv = stage_key[i];
            if constexpr (SRC_SCORES)
                pos = page_row ? page_row[(uint32_t)c / (uint32_t)P] * P + (int32_t)((uint32_t)c % (uint32_t)P)
                               : (int32_t)c;
            else
                pos = in_pos[(int64_t)r * in_ld + c];
        }
        if constexpr (FINAL) {
            idx[(int64_t)r * k + i] = pos;
        } else {
            out_key[(int64_t)r * out_ld + (int64_t)seg * k + i] = kv;
            out_pos[(int64_t)r * out_ld + (int64_t)seg * k + i] = pos;
        }
    }
}

// Candidates per row after level 1 and after one more level; row strides are rounded up to 4.
static inline int64_t round4(int64_t x) { return (x + 3) & ~(int64_t)3; }
static void topk2_sizes(int64_t n_cols, int k, int64_t &n_seg, int64_t &l0, int64_t &l1)
{
    n_seg = (n_cols + kSeg - 1) / kSeg;
    l0 = n_seg * k;
    l1 = ((l0 + kSeg - 1) / kSeg) * k;
}

size_t topk2_workspace_bytes(int n_rows, int64_t n_cols, int k)
{
    int64_t n_seg, l0, l1;
    topk2_sizes(n_cols, k, n_seg, l0, l1);
    if (n_seg <= 1)
        return 0;
    return 2 * align_up((size_t)n_rows * round4(l0) * 4) + 2 * align_up((size_t)n_rows * round4(l1) * 4);
}

bool topk_two_level(int k) { return k >= 1 && k <= kMaxLocalK; }

static hipError_t launch_topk2(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages,
                               int M, int P, int k, int32_t *idx, void *ws, RowGate gate, hipStream_t stream)
{
    int64_t n_seg, l0, l1;
    topk2_sizes(n_cols, k, n_seg, l0, l1);
    if (n_seg <= 1) {
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, true, true>), dim3(1, n_rows), dim3(kSegThreads), 0,
                           stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k, nullptr, nullptr, 0, idx,
                           gate.row_mode, gate.want);
        return hipGetLastError();
    }
    // Two candidate buffers (key, position) with row strides lda >= l0 and ldb >= l1, used in turn.
    const int64_t lda = round4(l0), ldb = round4(l1);
    char *p = (char *)ws;
    uint32_t *key_a = (uint32_t *)p;
    p += align_up((size_t)n_rows * lda * 4);
    int32_t *pos_a = (int32_t *)p;
    p += align_up((size_t)n_rows * lda * 4);
    uint32_t *key_b = (uint32_t *)p;
    p += align_up((size_t)n_rows * ldb * 4);
    int32_t *pos_b = (int32_t *)p;
    hipLaunchKernelGGL((topk_level_kernel<kSegThreads, true, false>), dim3((unsigned)n_seg, n_rows),
                       dim3(kSegThreads), 0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k, key_a,
                       pos_a, lda, nullptr, gate.row_mode, gate.want);
    int64_t n_in = l0;
    bool in_a = true;
    while (n_in > kSeg) {  // reduce the candidate lists further
        const int64_t segs = (n_in + kSeg - 1) / kSeg;
        const int64_t n_out = segs * k;
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, false, false>), dim3((unsigned)segs, n_rows),
                           dim3(kSegThreads), 0, stream, nullptr, 0, n_in, nullptr, 0, 1, in_a ? key_a : key_b,
                           in_a ? pos_a : pos_b, in_a ? lda : ldb, k, in_a ? key_b : key_a, in_a ? pos_b : pos_a,
                           in_a ? ldb : lda, nullptr, gate.row_mode, gate.want);
        n_in = n_out;
        in_a = !in_a;
    }
    const uint32_t *fk = in_a ? key_a : key_b;
    const int32_t *fp = in_a ? pos_a : pos_b;
    const int64_t fld = in_a ? lda : ldb;
    hipLaunchKernelGGL((topk_level_kernel<kSegThreads, false, true>), dim3(1, n_rows), dim3(kSegThreads), 0, stream,
                       nullptr, 0, n_in, nullptr, 0, 1, fk, fp, fld, k, nullptr, nullptr, 0, idx, gate.row_mode,
                       gate.want);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------- host

hipError_t launch_topk_geo(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M,
                           int P, int k, int32_t *idx, void *ws_ptr, TopkGeom geo, bool pass0_done, RowGate gate,
                           hipStream_t stream)
{
    if (n_rows == 0)
        return hipSuccess;
    if (topk_two_level(k))
        return launch_topk2(n_rows, scores, ld, n_cols > 0 ? n_cols : 0, pages, M, P, k, idx, ws_ptr, gate, stream);
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
