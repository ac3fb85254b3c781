// topk_block.hpp -- the block-level exact selection shared by the top-K levels (topk.hip) and the
// fused scoring + first-level selection (index_score.hip): a block holds its keys in registers and
// picks its best k under (key desc, position asc) by radix select over the keys' own range on LDS
// histograms, finished by a one-wave ranking, then writes the picks to LDS in position order.  (Keys:
// order-preserving images of the scores, 0 = not a candidate.)
#pragma once
#include "lsa_dev.hpp"

namespace lsa {

constexpr int kBins = 2048;

constexpr int kDigitBits = 11;  // digits of at most 11 bits: 2048 bins

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

// The result of a selection, as thresholds on the whole key: a key x is picked when x >= t_gt, and of the
// keys equal to t_eq the first k_rem in position order are picked (t_eq = 0xffffffff, which no key
// takes, when there are none to rank).  Every candidate is picked when `all` (t_gt = 1).
struct Selection {
    uint32_t t_gt;
    uint32_t t_eq;
    uint32_t k_rem;
    bool all;
};

// Radix select of the block's best k among the non-zero keys (0 = not a candidate), on the range the
// keys actually take: every candidate lies in [kmin, kmax], so the search keeps an interval
// [lo, lo + 2^s) that holds the k-th key, starting from lo = kmin and the least s with
// kmax - kmin < 2^s, and each pass splits it into 2^11 bins by the digit (x - lo) >> (s - 11).
// (Indexer scores of one block span a few binades: digits of a common bit prefix would be mostly
// exponent bits and put the keys into a few bins, serialising the histogram atomics, and need a second
// pass every time.)  Once the bin that holds the k-th key holds at most 64 keys, one wave ranks them.
// The digit histograms live in LDS as kCopies interleaved copies (bin b, copy c at hist[kCopies b + c];
// lane l adds to copy l % kCopies), so the atomics on a crowded bin go to consecutive banks.  In the
// first pass the keys outside the interval (the zeros) add to a per-lane dummy word (no branch per
// key); later passes count only the keys of the previous bin, by a branch.
constexpr int kCopies = 2;
constexpr int kHistWords = kBins * kCopies + kWave;  // + one dummy word per lane
constexpr int kStageWords = 2 * (kMaxLocalK + kWave);
constexpr int kLdsWords = kHistWords > kStageWords ? kHistWords : kStageWords;

// A thread's count of candidates, its least candidate key less one (0xffffffff when it has none: the
// key 0 wraps round) and its largest key, gathered key by key.
struct KeyStats {
    uint32_t cnt = 0u, low_m1 = 0xffffffffu, high = 0u;
    __device__ __attribute__((always_inline)) void add(uint32_t x)
    {
        cnt += x != 0u ? 1u : 0u;
        low_m1 = min(low_m1, x - 1u);
        high = max(high, x);
    }
};

// The selection on keys whose per-thread statistics are given (st: this thread's keys').
template <int NT, int VPT>
__device__ __attribute__((always_inline)) Selection block_select(const uint32_t (&key)[VPT], uint32_t k, KeyStats st,
                                                                 uint32_t *hist, uint32_t *scratch, int *s_d,
                                                                 uint32_t *s_above, uint32_t *s_bin)
{
    Selection sel{1u, 0xffffffffu, k, false};
    uint32_t total = st.cnt, kmin = st.low_m1, kmax = st.high;
    block_reduce3<NT>(total, kmin, kmax, scratch);
    kmin += 1u;  // (a candidate exists whenever it is used below)
    if (total <= k) {
        sel.all = true;
        return sel;
    }
    if (kmin == kmax) {  // all candidates equal: the first k in position order
        sel.t_gt = kmin + 1u, sel.t_eq = kmin;
        return sel;
    }
    uint32_t lo = kmin;
    int s = 32 - __clz(kmax - kmin);  // kmax - lo < 2^s, 1 <= s <= 32
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t copy = lane % kCopies, dummy = kBins * kCopies + lane;
    constexpr int kPer = kBins / NT;  // bins owned by a thread in the suffix scan
    // Cleared once here; afterwards every pass clears the words it has read.
    for (int i = threadIdx.x; i < kBins * kCopies / 4; i += NT)
        reinterpret_cast<uint4 *>(hist)[i] = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    // x in [lo, lo + 2^s) after the first pass (s <= 21): x - lo < 2^s in 32 bits, since for a key below
    // lo (a zero too) x - lo wraps to at least 2^32 - lo >= 2^23 (lo <= 0xff800000, the largest
    // candidate key)
    auto inside = [](uint32_t x, uint32_t l, int w) __attribute__((always_inline)) { return x - l < (1u << w); };
    for (int pass = 0; pass < 3; ++pass) {
        const int width = min(kDigitBits, s);
        const int shift = s - width;
        if (pass == 0) {
            // every candidate lies in the first interval: only the zeros stay out
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                uint32_t x = key[m];
                asm volatile("" : "+v"(x));  // (opaque: keeps each compare mask in its own iteration)
                atomicAdd(&hist[x != 0u ? kCopies * ((x - lo) >> shift) + copy : dummy], 1u);
            }
        } else {
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                uint32_t x = key[m];
                asm volatile("" : "+v"(x));  // (as above)
                if (inside(x, lo, s))
                    atomicAdd(&hist[kCopies * ((x - lo) >> shift) + copy], 1u);
            }
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
        lo += (uint32_t)d << shift;
        s = shift;
        if (bin == sel.k_rem) {  // the bin is picked whole: every key >= lo
            sel.t_gt = lo;
            return sel;
        }
        if (s == 0) {  // the bin is one key value: ties, ranked by position
            sel.t_gt = lo + 1u, sel.t_eq = lo;
            return sel;
        }
        if (bin <= (uint32_t)kWave) {
            // One wave ranks the bin's keys, gathered in the histogram words (all zero after a pass;
            // hist[kWave] counts them).  The k_rem-th largest of them, T, is the threshold: the keys
            // above T are picked, and of those equal to T the first k_rem - (the bin's keys above T).
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                uint32_t x = key[m];
                asm volatile("" : "+v"(x));  // (as above)
                if (inside(x, lo, s)) {
                    const uint32_t slot = atomicAdd(&hist[kWave], 1u);
                    if (slot < (uint32_t)kWave)  // (always: the bin holds at most 64 keys)
                        hist[slot] = x;
                }
            }
            __syncthreads();
            if (threadIdx.x < kWave) {
                const uint32_t v = lane < bin ? hist[lane] : 0u;  // (0 lies below every key of the bin)
                uint32_t gt = 0, ge = 0;
                for (int j = 0; j < (int)bin; ++j) {
                    const uint32_t u = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
                    gt += u > v ? 1u : 0u;
                    ge += u >= v ? 1u : 0u;
                }
                // T: a key of the bin with gt < k_rem <= ge (1 <= k_rem < bin; the lanes past the bin
                // have gt = bin); every key equal to T is taken when ge = k_rem
                const uint64_t hit = __ballot(lane < bin && gt < sel.k_rem && sel.k_rem <= ge);
                if (lane == (uint32_t)(__ffsll((long long)hit) - 1))
                    *s_above = v, *s_bin = gt, *s_d = ge == sel.k_rem ? 1 : 0;
            }
            __syncthreads();
            const uint32_t t = *s_above;
            sel.k_rem -= *s_bin;
            if (*s_d)
                sel.t_gt = t;  // (no ties to rank)
            else
                sel.t_gt = t + 1u, sel.t_eq = t;
            __syncthreads();  // (the callers' next LDS writes may reuse these words)
            return sel;
        }
    }
    return sel;  // (not reached: s reaches 0 within three passes)
}

template <int NT, int VPT>
__device__ __attribute__((always_inline)) Selection block_select(const uint32_t (&key)[VPT], uint32_t k,
                                                                 uint32_t *hist, uint32_t *scratch, int *s_d,
                                                                 uint32_t *s_above, uint32_t *s_bin)
{
    KeyStats st;
#pragma unroll
    for (int m = 0; m < VPT; ++m)
        st.add(key[m]);
    return block_select<NT, VPT>(key, k, st, hist, scratch, s_d, s_above, s_bin);
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
    //   (0xffffffff is a NaN pattern, mapped to key 0: no key equals it.)
    const uint32_t t_gt = sel.t_gt, t_eq = sel.t_eq;
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

}  // namespace lsa
