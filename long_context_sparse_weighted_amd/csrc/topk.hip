// topk.hip -- exact arg-topK ([paper] §2.2 Eq. 2; SI middle region of [review] §2.1; HI stage 2 of
// [paper] §3.3, which selects Ksparse tokens among recalled pages).
//
// Keys are the order-preserving 32-bit images of the scores (-0 folded onto +0); -inf and NaN are
// not candidates and map to key 0.  The selection runs in levels.  A block of 512 threads holds a
// segment of 16384 keys in registers (thread t holds positions 32 t .. 32 t + 31 of the segment; a
// whole row of at most 4096 columns goes to one block of 256 threads x 16 keys, a final list of at
// most 8192 candidates to 512 threads x 16) and picks its best k under (key desc, position asc) by
// MSB-first radix select over the range its keys take: from [kmin, kmax], each pass splits the
// interval holding the k-th key into 2^11 bins, counted in an LDS histogram whose suffix sums locate
// the bin of the k-th key; keys above that bin are picked, and once the bin holds at most 64 keys one
// wave ranks them exactly; ties at the k-th key's value take the lowest positions.
// The picks are written in position order.  The first level cuts each row into segments of 16384
// scores and writes every segment's picks as a candidate list (key, position): the row's top k is
// among them, since an element with fewer than k better elements in its row has fewer than k
// better elements in its segment.  Further levels do the same on the candidate lists (whose order
// is still position order) until one segment per row remains, whose picks are the result.  Scores
// are read once; there are no global atomics and no fences, and the result is exact and bitwise
// deterministic.
#include "lsa_kernels.hpp"
#include "topk_block.hpp"

namespace lsa {

#ifndef LSA_TOPK_THREADS
#define LSA_TOPK_THREADS 512
#endif
constexpr int kSeg = 16384;                     // keys per segment (one block)
constexpr int kSegThreads = LSA_TOPK_THREADS;
constexpr int kVpt = kSeg / kSegThreads;        // keys per thread
constexpr int kSmallThreads = 256;
constexpr int kSmallVpt = 16;                   // a row of at most 4096 columns: one block of 256 x 16
constexpr int kFinalVpt = 16;                   // a final candidate list of at most 8192: 512 x 16
constexpr int64_t kListSeg = kSeg;              // candidates per segment of the non-final list levels


// One level.  SRC_SCORES: segment `seg` of row r is columns [seg * 64 NT, ...) of the scores (page
// mapped when pages is given; P is a multiple of 16, so 16 aligned columns share a page);
// otherwise candidates [seg * 64 NT, ...) of row r's list of n_in.  FINAL: the picks (positions)
// go to idx[r][0 .. k), padded with -1; otherwise to the next list at [seg * k, seg * k + k),
// padded with key 0.
// A first level over a score matrix (every block of a prefill batch) is bound by the latency of its
// barrier-separated radix passes, not by HBM: capped at 80 VGPRs, three of its 512-thread blocks share
// a CU instead of two (8192 rows x 139,264 scores: 2.16 -> 1.81 ms).
constexpr int kScoreLevelWavesPerEU = 6;

template <int NT, int VPT, bool SRC_SCORES, bool FINAL>
__global__ __launch_bounds__(NT, SRC_SCORES && VPT == 32 ? kScoreLevelWavesPerEU : 1) void topk_level_kernel(
    const float *__restrict__ scores, int64_t ld, int64_t n_in, const int32_t *__restrict__ pages, int M, int P,
    const uint32_t *__restrict__ in_key, const int32_t *__restrict__ in_pos, int64_t in_ld, int k,
    uint32_t *__restrict__ out_key, int32_t *__restrict__ out_pos, int64_t out_ld, int32_t *__restrict__ idx,
    const uint8_t *row_mode, int want, ListCount cnt, int level)
{
    const int seg = blockIdx.x, r = blockIdx.y;
    if (row_mode && row_mode[r] != want)
        return;
    if constexpr (!SRC_SCORES) {
        if (cnt.on) {
            // this row's own list length at this level (its first level wrote fused_row_lists lists)
            int64_t m = fused_row_lists(cnt.rows, r, cnt.k_sink, cnt.k_swa, cnt.cols) * k;
            for (int l = 0; l < level; ++l)
                m = (m + kListSeg - 1) / kListSeg * k;  // each level keeps k per segment of kListSeg
            n_in = m < n_in ? m : n_in;
            if (!FINAL && (int64_t)seg * (VPT * NT) >= n_in)
                return;  // past the row's lists: nothing to read and nothing the next level reads
        }
    }
    // LDS: the histograms, reused afterwards as the staging area of the picks.
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];
    __shared__ uint32_t scratch[3 * NT / kWave];
    __shared__ int s_d;
    __shared__ uint32_t s_above, s_bin;
    const int64_t seg_base = (int64_t)seg * (VPT * NT);
    const int64_t base = seg_base + (int64_t)VPT * threadIdx.x;  // this thread's first element
    const int32_t *page_row = pages ? pages + (int64_t)r * M : nullptr;
    // page slot of column c (c < M P < 2^31): a shift for a power-of-two page size
    const int p_shift = (P & (P - 1)) == 0 ? __builtin_ctz((unsigned)P) : -1;
    auto slot_of = [&](uint32_t c) { return p_shift >= 0 ? c >> p_shift : c / (uint32_t)P; };
    uint32_t key[VPT];
    if constexpr (SRC_SCORES) {
        const float *row = scores + (int64_t)r * ld;
        if (base + VPT <= n_in && (ld & 3) == 0 && ((uintptr_t)scores & 15) == 0) {
            const float4 *src = reinterpret_cast<const float4 *>(row + base);
#pragma unroll
            for (int q = 0; q < VPT / 4; ++q) {
                const float4 v = src[q];
                key[4 * q] = candidate_key(v.x);
                key[4 * q + 1] = candidate_key(v.y);
                key[4 * q + 2] = candidate_key(v.z);
                key[4 * q + 3] = candidate_key(v.w);
            }
        } else if ((ld & 3) == 0 && ((uintptr_t)scores & 15) == 0) {
            // A partial segment: whole float4 where it lies below n_in, single elements only in the
            // float4 that straddles it.
            const float4 *src = reinterpret_cast<const float4 *>(row + base);
#pragma unroll
            for (int q = 0; q < VPT / 4; ++q) {
                const int64_t c = base + 4 * q;
                float4 v = float4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                if (c + 4 <= n_in) {
                    v = src[q];
                } else if (c < n_in) {
                    v.x = row[c];
                    v.y = c + 1 < n_in ? row[c + 1] : -INFINITY;
                    v.z = c + 2 < n_in ? row[c + 2] : -INFINITY;
                }
                key[4 * q] = candidate_key(v.x);
                key[4 * q + 1] = candidate_key(v.y);
                key[4 * q + 2] = candidate_key(v.z);
                key[4 * q + 3] = candidate_key(v.w);
            }
        } else {
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                const int64_t c = base + m;
                const float v = c < n_in ? row[c] : -INFINITY;
                key[m] = candidate_key(v);
            }
        }
        if (page_row) {
#pragma unroll
            for (int q = 0; q < VPT / 16; ++q) {
                const int64_t c = base + 16 * q;
                const bool ok = c < n_in && page_row[slot_of((uint32_t)c)] >= 0;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    key[16 * q + i] = ok ? key[16 * q + i] : 0u;
            }
        }
    } else {
        const uint32_t *src = in_key + (int64_t)r * in_ld;
        if (base + VPT <= n_in) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(src + base);
#pragma unroll
            for (int q = 0; q < VPT / 4; ++q) {
                const uint4 v = s4[q];
                key[4 * q] = v.x, key[4 * q + 1] = v.y, key[4 * q + 2] = v.z, key[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < VPT; ++m)
                key[m] = base + m < n_in ? src[base + m] : 0u;
        }
    }
    const Selection sel = block_select<NT, VPT>(key, (uint32_t)k, lds, scratch, &s_d, &s_above, &s_bin);
    uint32_t *stage_key = lds, *stage_li = lds + kMaxLocalK + kWave;
    __syncthreads();  // the histograms are no longer read
    const uint32_t n_sel = block_emit<NT, VPT>(key, sel, scratch, stage_key, stage_li, (uint32_t)(VPT * threadIdx.x));
    __syncthreads();
    // Copy-out in slot order (coalesced), with positions computed for the picks only.
    for (int i = threadIdx.x; i < k; i += NT) {
        int32_t pos = -1;
        uint32_t kv = 0;
        const int64_t c = seg_base + stage_li[i];
        if ((uint32_t)i < n_sel && c < n_in) {  // (a pick is always below n_in: keys past it are 0)
            kv = stage_key[i];
            if constexpr (SRC_SCORES)
                pos = page_row ? page_row[slot_of((uint32_t)c)] * P + (int32_t)((uint32_t)c - slot_of((uint32_t)c) * (uint32_t)P)
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

// Two candidate buffers (key, position) with row strides lda >= l0 and ldb >= l1, used in turn.
struct TopkLists {
    uint32_t *key_a, *key_b;
    int32_t *pos_a, *pos_b;
    int64_t lda, ldb;
};

static TopkLists topk_lists(void *ws, int n_rows, int64_t l0, int64_t l1)
{
    TopkLists t;
    t.lda = round4(l0);
    t.ldb = round4(l1);
    char *p = (char *)ws;
    t.key_a = (uint32_t *)p;
    p += align_up((size_t)n_rows * t.lda * 4);
    t.pos_a = (int32_t *)p;
    p += align_up((size_t)n_rows * t.lda * 4);
    t.key_b = (uint32_t *)p;
    p += align_up((size_t)n_rows * t.ldb * 4);
    t.pos_b = (int32_t *)p;
    return t;
}

// The levels after the first: lists of n_in candidates per row in t's A buffers, reduced segment by
// segment until one remains, whose picks go to idx.
static hipError_t run_list_levels(int n_rows, int64_t n_in, int k, const TopkLists &t, int32_t *idx, RowGate gate,
                                  ListCount cnt, hipStream_t stream)
{
    bool in_a = true;
    int level = 0;
    while (n_in > kSeg) {  // reduce the candidate lists further
        const int64_t segs = (n_in + kSeg - 1) / kSeg;
        const int64_t n_out = segs * k;
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, false, false>), dim3((unsigned)segs, n_rows),
                           dim3(kSegThreads), 0, stream, nullptr, 0, n_in, nullptr, 0, 1, in_a ? t.key_a : t.key_b,
                           in_a ? t.pos_a : t.pos_b, in_a ? t.lda : t.ldb, k, in_a ? t.key_b : t.key_a,
                           in_a ? t.pos_b : t.pos_a, in_a ? t.ldb : t.lda, nullptr, gate.row_mode, gate.want, cnt,
                           level);
        n_in = n_out;
        in_a = !in_a;
        ++level;
    }
    const uint32_t *fk = in_a ? t.key_a : t.key_b;
    const int32_t *fp = in_a ? t.pos_a : t.pos_b;
    const int64_t fld = in_a ? t.lda : t.ldb;
    if (n_in <= kSegThreads * kFinalVpt)  // (8 segments' picks at 128K columns): half the keys per thread
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kFinalVpt, false, true>), dim3(1, n_rows), dim3(kSegThreads),
                           0, stream, nullptr, 0, n_in, nullptr, 0, 1, fk, fp, fld, k, nullptr, nullptr, 0, idx,
                           gate.row_mode, gate.want, cnt, level);
    else
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, false, true>), dim3(1, n_rows), dim3(kSegThreads), 0,
                           stream, nullptr, 0, n_in, nullptr, 0, 1, fk, fp, fld, k, nullptr, nullptr, 0, idx,
                           gate.row_mode, gate.want, cnt, level);
    return hipGetLastError();
}

size_t topk_workspace_bytes(int n_rows, int64_t n_cols, int k)
{
    int64_t n_seg, l0, l1;
    topk2_sizes(n_cols > 0 ? n_cols : 1, k, n_seg, l0, l1);
    if (n_seg <= 1)
        return 0;
    return 2 * align_up((size_t)n_rows * round4(l0) * 4) + 2 * align_up((size_t)n_rows * round4(l1) * 4);
}

hipError_t launch_topk(int n_rows, const float *scores, int64_t ld, int64_t n_cols, const int32_t *pages, int M, int P,
                       int k, int32_t *idx, void *ws, RowGate gate, hipStream_t stream)
{
    if (k < 1 || k > kMaxLocalK)
        return hipErrorInvalidValue;
    if (n_rows == 0)
        return hipSuccess;
    if (n_cols < 0)
        n_cols = 0;
    int64_t n_seg, l0, l1;
    topk2_sizes(n_cols, k, n_seg, l0, l1);
    if (n_seg <= 1) {
        // One segment per row: with at most 4096 columns, 16 keys per thread (a quarter of the per-key
        // work of the 16384-column segment).
        if (n_cols <= kSmallVpt * kSmallThreads)
            hipLaunchKernelGGL((topk_level_kernel<kSmallThreads, kSmallVpt, true, true>), dim3(1, n_rows),
                               dim3(kSmallThreads), 0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k,
                               nullptr, nullptr, 0, idx, gate.row_mode, gate.want, ListCount{}, 0);
        else if (n_cols <= kFinalVpt * kSegThreads)  // at most 8192 columns (the page recall at 1M, P = 128)
            hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kFinalVpt, true, true>), dim3(1, n_rows),
                               dim3(kSegThreads), 0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k,
                               nullptr, nullptr, 0, idx, gate.row_mode, gate.want, ListCount{}, 0);
        else
            hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, true, true>), dim3(1, n_rows), dim3(kSegThreads),
                               0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k, nullptr, nullptr, 0,
                               idx, gate.row_mode, gate.want, ListCount{}, 0);
        return hipGetLastError();
    }
    TopkLists t = topk_lists(ws, n_rows, l0, l1);
    hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, true, false>), dim3((unsigned)n_seg, n_rows),
                       dim3(kSegThreads), 0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k, t.key_a,
                       t.pos_a, t.lda, nullptr, gate.row_mode, gate.want, ListCount{}, 0);
    return run_list_levels(n_rows, l0, k, t, idx, gate, ListCount{}, stream);
}

size_t topk_lists_workspace_bytes(int n_rows, int64_t n_seg, int k)
{
    const int64_t l0 = n_seg * k, l1 = ((l0 + kSeg - 1) / kSeg) * k;
    return 2 * align_up((size_t)n_rows * round4(l0) * 4) + 2 * align_up((size_t)n_rows * round4(l1) * 4);
}

void topk_first_lists(void *ws, int n_rows, int64_t n_seg, int k, uint32_t **key, int32_t **pos, int64_t *ld)
{
    const int64_t l0 = n_seg * k, l1 = ((l0 + kSeg - 1) / kSeg) * k;
    const TopkLists t = topk_lists(ws, n_rows, l0, l1);
    *key = t.key_a;
    *pos = t.pos_a;
    *ld = t.lda;
}

hipError_t launch_topk_lists(int n_rows, int64_t n_seg, int k, void *ws, int32_t *idx, RowGate gate, ListCount cnt,
                             hipStream_t stream)
{
    if (k < 1 || k > kMaxLocalK)
        return hipErrorInvalidValue;
    if (n_rows == 0)
        return hipSuccess;
    const int64_t l0 = n_seg * k, l1 = ((l0 + kSeg - 1) / kSeg) * k;
    return run_list_levels(n_rows, l0, k, topk_lists(ws, n_rows, l0, l1), idx, gate, cnt, stream);
}

}  // namespace lsa
