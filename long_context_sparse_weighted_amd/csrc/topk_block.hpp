// topk_block.hpp -- the block-level exact selection shared by the top-K levels (topk.hip) and the
// fused scoring + first-level selection (index_score.hip): a block holds its keys in registers and
// picks its best k under (key desc, position asc) by MSB-first radix select on LDS histograms, then
// writes the picks to LDS in position order.  (Keys: order-preserving images of the scores, 0 = not a
// candidate.)
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

}  // namespace lsa
