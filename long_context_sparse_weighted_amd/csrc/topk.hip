// topk.hip -- exact arg-topK by MSB-first radix select ([paper] §2.2 Eq. 2; SI middle region of
// [review] §2.1; HI stage 2 of [paper] §3.3, which selects Ksparse tokens among recalled pages).
//
// Every candidate column c of a row gets a unique 64-bit key
//     key = (order(score) << pos_bits) | (n_cols - 1 - c)
// so that "larger key" is exactly "better" under (score desc, position asc) and no two keys tie.
// The K-th largest key is found digit by digit, 11 bits per pass (2048-bin histograms):
//   pass p: every block of a row histograms the digit of the keys that still match the prefix
//           fixed so far (LDS histogram, merged into the row's global histogram with integer
//           atomics); the last block to finish (atomic ticket) scans the histogram from the top
//           digit, fixes the digit that holds the K-th key, and stops the search as soon as that
//           digit's bin is taken whole.
//   collect: every key whose fixed top bits are >= the prefix is selected (exactly
//            min(K, #candidates) of them); positions are appended with wave-aggregated atomics.
//   sort:    one block per row sorts its <= K positions ascending (bitonic, LDS), pads with -1.
// Integer atomics only, so the result is bitwise deterministic.  Rows are split over many
// blocks, so a handful of 1M-candidate decode rows still fill the chip.
#include "lsa_kernels.hpp"

namespace lsa {

constexpr int kBins = 2048;
constexpr int kDigit = 11;
constexpr int kMaxK = 4096;
constexpr int kPassThreads = 256;
constexpr int kPassElems = 16;  // per thread per block

struct TopkState {
    unsigned long long prefix;  // fixed top `consumed` bits of the K-th key
    uint32_t consumed;          // number of fixed top bits
    uint32_t k_rem;             // keys still to take inside the bin of `prefix`
    uint32_t done;              // 1: selection = { key : top(key, consumed) >= prefix }
    uint32_t ticket;            // blocks finished in this pass
    uint32_t out_count;         // positions collected
    uint32_t active;            // row takes part
    uint32_t pad[8];
};
static_assert(sizeof(TopkState) == 64, "state is one 64-byte slot per row");

struct TopkWs {
    TopkState *state;  // [n_rows]
    uint32_t *hist;    // [n_rows][kBins]
    int32_t *list;     // [n_rows][k]
};

static TopkWs carve(void *ws, int n_rows, int k)
{
    char *p = (char *)ws;
    TopkWs t;
    t.state = (TopkState *)p;
    p += align_up(sizeof(TopkState) * (size_t)n_rows);
    t.hist = (uint32_t *)p;
    p += align_up(sizeof(uint32_t) * kBins * (size_t)n_rows);
    t.list = (int32_t *)p;
    return t;
}

size_t topk_workspace_bytes(int n_rows, int k)
{
    return align_up(sizeof(TopkState) * (size_t)n_rows) + align_up(sizeof(uint32_t) * kBins * (size_t)n_rows) +
           align_up(sizeof(int32_t) * (size_t)k * n_rows);
}

__device__ inline unsigned long long make_key(float s, int64_t c, int64_t n_cols, int pos_bits)
{
    return ((unsigned long long)float_order_key(s) << pos_bits) | (unsigned long long)(n_cols - 1 - c);
}

__global__ void topk_init_kernel(TopkWs ws, int k, const uint8_t *row_mode, int want)
{
    const int r = blockIdx.x;
    TopkState *st = ws.state + r;
    const bool active = !row_mode || row_mode[r] == want;
    if (threadIdx.x == 0) {
        st->prefix = 0;
        st->consumed = 0;
        st->k_rem = (uint32_t)k;
        st->done = active ? 0u : 1u;
        st->ticket = 0;
        st->out_count = 0;
        st->active = active ? 1u : 0u;
    }
    uint32_t *h = ws.hist + (int64_t)r * kBins;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x)
        h[i] = 0;
}

__global__ __launch_bounds__(kPassThreads) void topk_pass_kernel(const float *__restrict__ scores, int64_t ld,
                                                                 int64_t n_cols, const int32_t *pages, int M, int P,
                                                                 int pos_bits, int pass, TopkWs ws)
{
    const int r = blockIdx.y;
    TopkState *st = ws.state + r;
    if (st->done)
        return;
    __shared__ uint32_t lh[kBins];
    __shared__ int is_last;
    const int T = 32 + pos_bits;
    const int hi_bit = T - kDigit * pass;                  // digit covers bits [shift, hi_bit)
    const int shift = hi_bit > kDigit ? hi_bit - kDigit : 0;
    const int width = hi_bit - shift;
    const unsigned long long prefix = st->prefix;
    const uint32_t consumed = st->consumed;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x)
        lh[i] = 0;
    __syncthreads();

    const float *row = scores + (int64_t)r * ld;
    const int32_t *page_row = pages ? pages + (int64_t)r * M : nullptr;
    const int64_t c0 = (int64_t)blockIdx.x * kPassThreads * kPassElems;
    const unsigned long long dmask = (1ull << width) - 1;
    const int lane = lane_id();
    // Load the whole batch first so the loads are all in flight together.
    float sv[kPassElems];
#pragma unroll
    for (int e = 0; e < kPassElems; ++e) {
        const int64_t c = c0 + (int64_t)e * kPassThreads + threadIdx.x;
        sv[e] = c < n_cols ? row[c] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < kPassElems; ++e) {
        const int64_t c = c0 + (int64_t)e * kPassThreads + threadIdx.x;
        bool want = false;
        uint32_t d = 0;
        if (c < n_cols && is_candidate(sv[e]) && (!page_row || page_row[c / P] >= 0)) {
            unsigned long long key = make_key(sv[e], c, n_cols, pos_bits);
            if (consumed == 0 || (key >> (T - consumed)) == prefix) {
                want = true;
                d = (uint32_t)((key >> shift) & dmask);
            }
        }
        // Scores of one row crowd into a few bins: lanes that share a digit add it once
        // (one LDS atomic per distinct digit, up to 8 of them); the rest add individually.
        for (int it = 0; it < 8; ++it) {
            unsigned long long act = __ballot(want);
            if (act == 0)
                break;
            const int leader = __ffsll((long long)act) - 1;
            const uint32_t dl = (uint32_t)__shfl((int)d, leader, kWave);
            const bool same = want && d == dl;
            const unsigned long long m = __ballot(same);
            if (lane == leader)
                atomicAdd(&lh[dl], (uint32_t)__popcll(m));
            if (same)
                want = false;
        }
        if (want)
            atomicAdd(&lh[d], 1u);
    }
    __syncthreads();
    uint32_t *gh = ws.hist + (int64_t)r * kBins;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x)
        if (lh[i])
            atomicAdd(&gh[i], lh[i]);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = atomicAdd(&st->ticket, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();

    // Last block of the row: read the merged histogram (coherently) and fix this digit.
    for (int i = threadIdx.x; i < kBins; i += blockDim.x)
        lh[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // Thread t owns the 8 bins [kBins-8(t+1), kBins-8t) scanned from the top.
    __shared__ uint32_t part[kPassThreads];
    const int t = threadIdx.x;
    uint32_t mine = 0;
    for (int i = 0; i < 8; ++i)
        mine += lh[kBins - 1 - (8 * t + i)];
    part[t] = mine;
    __syncthreads();
    // Inclusive suffix sums of the per-thread parts (from the top digit down), in one wave.
    __shared__ uint32_t above_part[kPassThreads];
    if (t < kWave) {
        uint32_t run = 0;
        for (int base = 0; base < kPassThreads; base += kWave) {
            uint32_t v = part[base + t];
            uint32_t incl = v;
            for (int o = 1; o < kWave; o <<= 1) {
                uint32_t y = (uint32_t)__shfl_up((int)incl, o, kWave);
                if (t >= o)
                    incl += y;
            }
            above_part[base + t] = run + incl - v;  // exclusive: sum of parts before this one
            run += (uint32_t)__shfl((int)incl, kWave - 1, kWave);
        }
    }
    __syncthreads();
    if (t == 0) {
        uint32_t k_rem = st->k_rem;
        const uint32_t total = above_part[kPassThreads - 1] + part[kPassThreads - 1];
        if (pass == 0 && total <= k_rem) {
            // At most K candidates: all of them are selected.
            st->done = 1;
        } else {
            // The part holding the K-th key: last part whose exclusive prefix is below k_rem.
            int lo = 0, hi = kPassThreads - 1;
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (above_part[mid] < k_rem)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            uint32_t above = above_part[lo];
            int d = kBins - 1 - 8 * lo;
            while (above + lh[d] < k_rem)
                above += lh[d--];
            k_rem -= above;
            st->prefix = (prefix << width) | (unsigned long long)d;
            st->consumed = consumed + (uint32_t)width;
            st->k_rem = k_rem;
            if (lh[d] == k_rem || shift == 0)
                st->done = 1;
        }
        st->ticket = 0;
    }
    __syncthreads();
    // Clear the row histogram for the next pass.
    for (int i = threadIdx.x; i < kBins; i += blockDim.x)
        gh[i] = 0;
}

__global__ __launch_bounds__(kPassThreads) void topk_collect_kernel(const float *__restrict__ scores, int64_t ld,
                                                                    int64_t n_cols, const int32_t *pages, int M,
                                                                    int P, int pos_bits, int k, TopkWs ws)
{
    const int r = blockIdx.y;
    TopkState *st = ws.state + r;
    if (!st->active)
        return;
    const int T = 32 + pos_bits;
    const unsigned long long prefix = st->prefix;
    const uint32_t consumed = st->consumed;
    const float *row = scores + (int64_t)r * ld;
    const int32_t *page_row = pages ? pages + (int64_t)r * M : nullptr;
    int32_t *list = ws.list + (int64_t)r * k;
    const int64_t c0 = (int64_t)blockIdx.x * kPassThreads * kPassElems;
    const int lane = lane_id();
    float sv[kPassElems];
#pragma unroll
    for (int e = 0; e < kPassElems; ++e) {
        const int64_t c = c0 + (int64_t)e * kPassThreads + threadIdx.x;
        sv[e] = c < n_cols ? row[c] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < kPassElems; ++e) {
        const int64_t c = c0 + (int64_t)e * kPassThreads + threadIdx.x;
        bool take = false;
        if (c < n_cols && is_candidate(sv[e]) && (!page_row || page_row[c / P] >= 0)) {
            unsigned long long key = make_key(sv[e], c, n_cols, pos_bits);
            take = consumed == 0 || (key >> (T - consumed)) >= prefix;
        }
        unsigned long long mask = __ballot(take);
        if (mask == 0)
            continue;
        uint32_t cnt = (uint32_t)__popcll(mask);
        int leader = __ffsll((long long)mask) - 1;
        uint32_t base = 0;
        if (lane == leader)
            base = atomicAdd(&st->out_count, cnt);
        base = __shfl(base, leader, kWave);
        if (take) {
            uint32_t slot = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1));
            int64_t pos = page_row ? (int64_t)page_row[c / P] * P + c % P : c;
            if (slot < (uint32_t)k)
                list[slot] = (int32_t)pos;
        }
    }
}

__global__ __launch_bounds__(512) void topk_sort_kernel(TopkWs ws, int k, int k_pow2, int32_t *__restrict__ idx)
{
    const int r = blockIdx.x;
    TopkState *st = ws.state + r;
    if (!st->active)
        return;
    __shared__ int32_t v[kMaxK];
    uint32_t cnt = st->out_count;
    if (cnt > (uint32_t)k)
        cnt = (uint32_t)k;
    const int32_t *list = ws.list + (int64_t)r * k;
    for (int i = threadIdx.x; i < k_pow2; i += blockDim.x)
        v[i] = i < (int)cnt ? list[i] : INT32_MAX;
    __syncthreads();
    for (int size = 2; size <= k_pow2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < k_pow2 / 2; i += blockDim.x) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool up = (lo & size) == 0;
                int32_t a = v[lo], b = v[hi];
                if ((a > b) == up) {
                    v[lo] = b;
                    v[hi] = a;
                }
            }
            __syncthreads();
        }
    }
    int32_t *out = idx + (int64_t)r * k;
    for (int i = threadIdx.x; i < k; i += blockDim.x)
        out[i] = i < (int)cnt ? v[i] : -1;
}

hipError_t launch_topk(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M, int P,
                       int k, int32_t *idx, void *ws_ptr, RowGate gate, hipStream_t stream)
{
    if (n_rows == 0)
        return hipSuccess;
    TopkWs ws = carve(ws_ptr, n_rows, k);
    int pos_bits = 1;
    while (pos_bits < 31 && (1ll << pos_bits) < n_cols)
        ++pos_bits;
    const int T = 32 + pos_bits;
    const int n_pass = (T + kDigit - 1) / kDigit;
    hipLaunchKernelGGL(topk_init_kernel, dim3(n_rows), dim3(256), 0, stream, ws, k, gate.row_mode, gate.want);
    const int64_t per_block = (int64_t)kPassThreads * kPassElems;
    const int64_t n_cols_eff = n_cols > 0 ? n_cols : 1;
    dim3 grid((unsigned)((n_cols_eff + per_block - 1) / per_block), (unsigned)n_rows);
    if (n_cols > 0) {
        for (int p = 0; p < n_pass; ++p)
            hipLaunchKernelGGL(topk_pass_kernel, grid, dim3(kPassThreads), 0, stream, scores, ld, n_cols, pages, M, P,
                               pos_bits, p, ws);
        hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kPassThreads), 0, stream, scores, ld, n_cols, pages, M, P,
                           pos_bits, k, ws);
    }
    int k_pow2 = 1;
    while (k_pow2 < k)
        k_pow2 <<= 1;
    hipLaunchKernelGGL(topk_sort_kernel, dim3(n_rows), dim3(512), 0, stream, ws, k, k_pow2, idx);
    return hipGetLastError();
}

}  // namespace lsa
