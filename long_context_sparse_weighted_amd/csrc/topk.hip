// topk.hip -- exact arg-topK ([paper] §2.2 Eq. 2; SI middle region of [review] §2.1; HI stage 2 of
// [paper] §3.3, which selects Ksparse tokens among recalled pages).
//
// Keys are the order-preserving 32-bit images of the scores (-0 folded onto +0); -inf and NaN are
// not candidates and map to key 0.  The selection runs in levels.  A block of 512 threads holds a
// segment of 16384 keys in registers (thread t holds positions 32 t .. 32 t + 31 of the segment; a
// whole row of at most 4096 columns goes to one block of 256 threads x 16 keys, a final list of at
// most 8192 candidates to 512 threads x 16) and picks its best k under (key desc, position asc) by
// MSB-first radix select.  The bits the block's smallest and largest candidates share are fixed at
// once (every candidate shares them); the rest are taken in digits of at most 11 bits, each counted
// in an LDS histogram whose suffix sums locate the bin of the k-th key; keys above that bin are
// picked and, once all 32 bits are fixed, ties take the lowest positions.
// The picks are written in position order.  The first level cuts each row into segments of 16384
// scores and writes every segment's picks as a candidate list (key, position): the row's top k is
// among them, since an element with fewer than k better elements in its row has fewer than k
// better elements in its segment.  Further levels do the same on the candidate lists (whose order
// is still position order) until one segment per row remains, whose picks are the result.  Scores
// are read once; there are no global atomics and no fences, and the result is exact and bitwise
// deterministic.
#include "lsa_kernels.hpp"

namespace lsa {

constexpr int kBins = 2048;

constexpr int kDigitBits = 11;  // digits of at most 11 bits: 2048 bins

#ifndef LSA_TOPK_THREADS
#define LSA_TOPK_THREADS 512
#endif
constexpr int kSeg = 16384;                     // keys per segment (one block)
constexpr int kSegThreads = LSA_TOPK_THREADS;
constexpr int kVpt = kSeg / kSegThreads;        // keys per thread
constexpr int kSmallThreads = 256;
constexpr int kSmallVpt = 16;                   // a row of at most 4096 columns: one block of 256 x 16
constexpr int kFinalVpt = 16;                   // a final candidate list of at most 8192: 512 x 16
constexpr int kMaxLocalK = 4096;

// Exclusive prefix sums over threads (in thread order) of two counters, and their totals.
// scratch: 2 * NT / 64 words of LDS.
template <int NT>
__device__ __attribute__((always_inline)) inline void block_scan2(uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb, uint32_t &ta, uint32_t &tb,
                                   uint32_t *scratch)
{
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
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

// Inclusive wave min / max by the same DPP row shifts and broadcasts as wave_incl_scan (lane 63 ends
// with the whole wave's); lanes without a source take the identity.
__device__ inline uint32_t wave_incl_min(uint32_t v)
{
    constexpr int kId = -1;  // 0xffffffff
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x111, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x112, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x114, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x118, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x142, 0xa, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, 0x143, 0xc, 0xf, false));
    return v;
}
__device__ inline uint32_t wave_incl_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
    return v;
}

// Block totals of a count, and the min / max of the keys (scratch: 3 * NT / 64 words of LDS).
template <int NT>
__device__ __attribute__((always_inline)) inline void block_reduce3(uint32_t &cnt, uint32_t &kmin, uint32_t &kmax,
                                                                    uint32_t *scratch)
{
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t ic = wave_incl_scan(cnt);
    kmin = wave_incl_min(kmin);
    kmax = wave_incl_max(kmax);
    if (lane == kWave - 1)
        scratch[w] = ic, scratch[NW + w] = kmin, scratch[2 * NW + w] = kmax;
    __syncthreads();
    uint32_t c = 0, lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        c += scratch[i];
        lo = min(lo, scratch[NW + i]);
        hi = max(hi, scratch[2 * NW + i]);
    }
    cnt = c, kmin = lo, kmax = hi;
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

template <int NT, int VPT>
__device__ __attribute__((always_inline)) Selection block_select(const uint32_t (&key)[VPT], uint32_t k,
                                                                 uint32_t *hist, uint32_t *scratch, int *s_d,
                                                                 uint32_t *s_above, uint32_t *s_bin)
{
    Selection sel{0u, 0, k, false, false};
    uint32_t total = 0, kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int m = 0; m < VPT; ++m) {
        const uint32_t x = key[m];
        total += x != 0 ? 1u : 0u;
        kmin = min(kmin, x != 0 ? x : 0xffffffffu);
        kmax = max(kmax, x);
    }
    block_reduce3<NT>(total, kmin, kmax, scratch);
    if (total <= k) {
        sel.all = true;
        return sel;
    }
    // Every candidate lies in [kmin, kmax], so it shares their common leading bits: the digits start
    // below them.  (The candidates of a later level, the best keys of their segments, sit in a narrow
    // range whose fixed top digits would pile them into a few bins.)
    sel.consumed = kmin == kmax ? 32 : __clz(kmin ^ kmax);
    sel.prefix = sel.consumed == 0 ? 0u : kmin >> (32 - sel.consumed);
    if (sel.consumed == 32)
        return sel;  // all candidates equal: the first k in position order
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t copy = lane % kCopies, dummy = kBins * kCopies + lane;
    constexpr int kPer = kBins / NT;  // bins owned by a thread in the suffix scan
    // Cleared once here; afterwards every pass clears the words it has read.
    for (int i = threadIdx.x; i < kBins * kCopies / 4; i += NT)
        reinterpret_cast<uint4 *>(hist)[i] = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int pass = 0; pass < 3 && sel.consumed < 32; ++pass) {
        const int width = min(kDigitBits, 32 - sel.consumed);
        const int shift = 32 - sel.consumed - width;
        const uint32_t dmask = (1u << width) - 1;
        // keys whose top `consumed` bits equal the prefix: (x & pmask) == pval (uniform scalars)
        const uint32_t pmask = sel.consumed == 0 ? 0u : ~0u << (32 - sel.consumed);
        const uint32_t pval = sel.consumed == 0 ? 0u : sel.prefix << (32 - sel.consumed);
        // Key 0 (not a candidate) can match only a zero prefix in pass 0, and then its digit is 0 while
        // a candidate's is not (a candidate's top 11 bits are never all zero -- that would make it -inf
        // or a NaN -- and with a zero prefix they all lie in the digit): its add goes to the dummy word
        // like those of keys outside the prefix, so segments padded with zeros do not pile their
        // atomics onto one bin.  (The test is on the digit, which changes with the pass, not on the
        // key: the compiler would keep 64 loop-invariant key tests in scalar registers.)
        const uint32_t keep0 = (pass != 0 || pval != 0u) ? 1u : 0u;
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const uint32_t x = key[m];
            const uint32_t d = (x >> shift) & dmask;
            const bool take = (x & pmask) == pval && (d | keep0) != 0u;
            atomicAdd(&hist[take ? kCopies * d + copy : dummy], 1u);
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
        sel.prefix = (sel.prefix << width) | (uint32_t)d;
        sel.consumed += width;
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
template <int NT, int VPT>
__device__ __attribute__((always_inline)) uint32_t block_emit(const uint32_t (&key)[VPT], const Selection &sel,
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
    const uint32_t dummy = kMaxLocalK + (uint32_t)lane_id();
    if (t_eq == 0xffffffffu) {
        // No ties to resolve (the usual case: the threshold bin was taken whole): the picks are the
        // keys >= t_gt, numbered in position order.
        uint32_t cg = 0;
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            // (an opaque copy: the compiler would otherwise keep all the compare masks of this loop
            // in scalar registers for the loop below, and spill them)
            uint32_t x = key[m];
            asm volatile("" : "+v"(x));
            cg += x >= t_gt ? 1u : 0u;
        }
        uint32_t bg, unused, tg, unused2;
        block_scan2<NT>(cg, 0, bg, unused, tg, unused2, scratch);
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const bool g = key[m] >= t_gt;
            const uint32_t slot = g ? bg : dummy;
            stage_key[slot] = key[m];
            stage_li[slot] = first_li + m;
            bg += g ? 1u : 0u;
        }
        return tg;
    }
    // Flags of this thread's keys as bit masks (bit m: key m).
    uint64_t gbits = 0, ebits = 0;
#pragma unroll
    for (int m = 0; m < VPT; ++m) {
        gbits |= (uint64_t)(key[m] >= t_gt ? 1u : 0u) << m;
        ebits |= (uint64_t)(key[m] == t_eq ? 1u : 0u) << m;
    }
    const uint32_t cg = (uint32_t)__popcll(gbits), ce = (uint32_t)__popcll(ebits);
    uint32_t bg, be, tg, te;
    block_scan2<NT>(cg, ce, bg, be, tg, te, scratch);
#pragma unroll
    for (int m = 0; m < VPT; ++m) {
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
template <int NT, int VPT, bool SRC_SCORES, bool FINAL>
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
                key[4 * q] = is_candidate(v.x) ? float_order_key(v.x) : 0u;
                key[4 * q + 1] = is_candidate(v.y) ? float_order_key(v.y) : 0u;
                key[4 * q + 2] = is_candidate(v.z) ? float_order_key(v.z) : 0u;
                key[4 * q + 3] = is_candidate(v.w) ? float_order_key(v.w) : 0u;
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
                key[4 * q] = is_candidate(v.x) ? float_order_key(v.x) : 0u;
                key[4 * q + 1] = is_candidate(v.y) ? float_order_key(v.y) : 0u;
                key[4 * q + 2] = is_candidate(v.z) ? float_order_key(v.z) : 0u;
                key[4 * q + 3] = is_candidate(v.w) ? float_order_key(v.w) : 0u;
            }
        } else {
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                const int64_t c = base + m;
                const float v = c < n_in ? row[c] : -INFINITY;
                key[m] = is_candidate(v) ? float_order_key(v) : 0u;
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
                               nullptr, nullptr, 0, idx, gate.row_mode, gate.want);
        else
            hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, true, true>), dim3(1, n_rows), dim3(kSegThreads),
                               0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k, nullptr, nullptr, 0,
                               idx, gate.row_mode, gate.want);
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
    hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, true, false>), dim3((unsigned)n_seg, n_rows),
                       dim3(kSegThreads), 0, stream, scores, ld, n_cols, pages, M, P, nullptr, nullptr, 0, k, key_a,
                       pos_a, lda, nullptr, gate.row_mode, gate.want);
    int64_t n_in = l0;
    bool in_a = true;
    while (n_in > kSeg) {  // reduce the candidate lists further
        const int64_t segs = (n_in + kSeg - 1) / kSeg;
        const int64_t n_out = segs * k;
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, false, false>), dim3((unsigned)segs, n_rows),
                           dim3(kSegThreads), 0, stream, nullptr, 0, n_in, nullptr, 0, 1, in_a ? key_a : key_b,
                           in_a ? pos_a : pos_b, in_a ? lda : ldb, k, in_a ? key_b : key_a, in_a ? pos_b : pos_a,
                           in_a ? ldb : lda, nullptr, gate.row_mode, gate.want);
        n_in = n_out;
        in_a = !in_a;
    }
    const uint32_t *fk = in_a ? key_a : key_b;
    const int32_t *fp = in_a ? pos_a : pos_b;
    const int64_t fld = in_a ? lda : ldb;
    if (n_in <= kSegThreads * kFinalVpt)  // (8 segments' picks at 128K columns): half the keys per thread
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kFinalVpt, false, true>), dim3(1, n_rows), dim3(kSegThreads),
                           0, stream, nullptr, 0, n_in, nullptr, 0, 1, fk, fp, fld, k, nullptr, nullptr, 0, idx,
                           gate.row_mode, gate.want);
    else
        hipLaunchKernelGGL((topk_level_kernel<kSegThreads, kVpt, false, true>), dim3(1, n_rows), dim3(kSegThreads), 0,
                           stream, nullptr, 0, n_in, nullptr, 0, 1, fk, fp, fld, k, nullptr, nullptr, 0, idx,
                           gate.row_mode, gate.want);
    return hipGetLastError();
}

}  // namespace lsa
