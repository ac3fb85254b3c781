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
#include "topk_block.hpp"

#include <type_traits>
#include <utility>

namespace lsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { kModeFlat = 0, kModePaged = 1, kModePageMean = 2 };

// ReLU as one IEEE maximum (v_maximum3_f32); fmaxf would first canonicalize its operand.
__device__ inline float relu(float x) { return __builtin_elementwise_maximum(x, 0.0f); }

// Pins values that were loaded from memory: the compiler waits for those loads here, before
// anything it cannot see (the counted LDS DMA) is in flight.
template <typename T>
__device__ inline void loaded_here(const T &v)
{
    asm volatile("" ::"v"(v));
}

// Per-row view of which key a column stands for.
struct ColMap {
    int64_t base;       // first key row of the sequence (k_idx) or of its means (k_mean)
    int64_t lo, hi;     // FLAT/PAGED: valid positions [lo, hi) = mid(t) cut at L
    int64_t nsb;        // PAGEMEAN: sub-blocks of the sequence
    int64_t last_page;  // PAGEMEAN: pages p <= last_page are causal and exist
    int G;              // PAGEMEAN: sub-blocks per page
    int P;              // PAGED: page size
    int p_shift;        // PAGED: log2(P) when P is a power of two, else -1
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
    m.p_shift = P > 0 && (P & (P - 1)) == 0 ? __builtin_ctz((unsigned)P) : -1;
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
        // the sub-blocks with a score, as a column range: those of the causal pages that exist
        m.lo = 0;
        m.hi = (m.last_page + 1) * m.G < m.nsb ? (m.last_page + 1) * m.G : m.nsb;
    }
    return m;
}

// Page slot of a page-mapped column (columns stay below M P < 2^31): a shift for the usual power-of-two
// page size instead of a division.
__device__ inline uint32_t page_slot(const ColMap &m, uint32_t c)
{
    return m.p_shift >= 0 ? c >> m.p_shift : c / (uint32_t)m.P;
}

// Key row of column c (or -1 when the column holds no score).
template <int MODE>
__device__ inline int64_t col_key(const ColMap &m, int64_t c)
{
    if (MODE == kModeFlat) {
        return (c >= m.lo && c < m.hi) ? m.base + c : -1;
    } else if (MODE == kModePaged) {
        const int64_t slot = page_slot(m, (uint32_t)c);
        if (slot >= m.M)
            return -1;
        int64_t pg = m.page_row[slot];
        if (pg < 0)
            return -1;
        int64_t s = pg * m.P + (c - slot * m.P);
        return (s >= m.lo && s < m.hi) ? m.base + s : -1;
    } else {
        return (c < m.nsb && c / m.G <= m.last_page) ? m.base + c : -1;
    }
}

// ------------------------------------------------------------------------------------------
// bf16 matrix-core kernels: 64 indexer heads x 128 dims.

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kTile = 16;          // keys per MFMA tile
constexpr int kWavesPerBlock = 4;

// Rows 16 G .. 16 G + 15 form group G.  A group is scored by the multi-row kernel when all of its
// rows exist and pass the row gate and its rows that lie inside their sequence (the others are empty
// rows, all -inf) share one sequence: the rows then read the same keys.
constexpr int kGroupRows = 16;

// The 16 rows are read at once, one per lane (lanes 16 .. 63 repeat them), and combined by ballots:
// the answer is the same in every wave.
__device__ inline bool group_uniform(const RowsDev &rows, const uint8_t *row_mode, int want, int grp)
{
    const int r0 = grp * kGroupRows;
    if (r0 + kGroupRows > rows.n_rows)
        return false;
    const int r = r0 + (lane_id() & (kGroupRows - 1));
    const bool gated_out = row_mode && row_mode[r] != want;
    const RowInfo ri = row_info(rows, r);
    if (__ballot(gated_out) != 0)
        return false;
    const uint64_t valid = __ballot(ri.valid);
    if (valid == 0)
        return true;
    const int32_t b = __shfl(ri.seq, __ffsll((long long)valid) - 1, kWave);
    return __ballot(ri.valid && ri.seq != b) == 0;
}

// The sequence of a group's rows that lie inside it (-1: every row of the group is empty).
__device__ inline int32_t group_seq(const RowsDev &rows, int grp)
{
    const RowInfo ri = row_info(rows, grp * kGroupRows + (lane_id() & (kGroupRows - 1)));
    const uint64_t valid = __ballot(ri.valid);
    return valid == 0 ? -1 : __shfl(ri.seq, __ffsll((long long)valid) - 1, kWave);
}

// ------------------------------------------------------------------------------------------
// Streaming bf16 kernel (rows scored one by one: decode, and page-mean rows of HI stage 1): a row's q
// (64 heads x 128 dims) stays in VGPRs as the A operands of v_mfma_f32_16x16x32_bf16 and the keys (or
// sub-block means) stream past it, moved by LDS DMA.  A DMA instruction reads 1 KB of whole 128-byte
// lines (4 key rows), where an MFMA operand load reads 64 bytes of each of 16 rows.  Each wave streams its own tiles through a private ring
// of S 4 KB buffers (up to S tiles in flight), so no barrier is needed.  Chunk c of key k of a tile
// sits at slot 16 k + (c ^ k): the 16 lanes reading one operand hit 16 different bank groups.
//
// The DMA is issued outside the compiler's view (it would otherwise wait for every DMA in flight
// before each LDS read); the waits are counted here instead.  Vector memory operations of a wave
// complete in issue order and every step issues exactly 4 DMA instructions (steps past the wave's
// last tile re-read that tile), so when tile k is due exactly the 4 (S - 1) DMA instructions of
// tiles k + 1 .. k + S - 1 follow its own; score stores in between only make "at most 4 (S - 1)
// outstanding" stricter.

// Two blocks per CU, each wave with a 4-deep ring (64 KB of LDS per block): two waves per SIMD then
// overlap one wave's DMA issue with the other's products (decode 32 x 128K: 188 us against 199 us
// with one block of 6-deep rings; 32 x 1M: 1479 against 1511 us).
#ifndef LSA_SCORE_RING
#define LSA_SCORE_RING 4
#endif
#ifndef LSA_SCORE_BLOCKS_PER_CU
#define LSA_SCORE_BLOCKS_PER_CU 2
#endif
constexpr int kScoreRing = LSA_SCORE_RING;

// 16 bytes per lane from global memory to LDS at lds_base + 16 * lane (lds_base wave-uniform).
// Cache policy of a key stream (STREAM): a row reads each key once, as whole lines, so the DMA is marked
// streaming (sc0 nt) and does not displace cached data -- unless other rows of the launch read the same
// keys: paged and page-mean rows of one sequence (the pages several rows of a prefill chunk recall, the
// means every row of a sequence scores) keep the default policy, under which those re-reads hit L2 and
// the last-level cache (kernels' KEEP; HI stage 2 of a 2048-row prefill chunk at 1M: 11.2 -> 8.0 ms).
// Rows that share nothing stream (flat decode under the default policy: 8 % slower; HI decode of 8
// sequences with B = 8: 10 % slower).
template <bool STREAM>
__device__ inline void dma_16(const void *src, uint32_t lds_base)
{
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc0 nt" ::"v"(src),
                     "s"(lds_base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
                     : "memory", "m0");
}

// The same from a wave-uniform base (SGPR pair) plus a per-lane 32-bit byte offset: no per-lane
// 64-bit address arithmetic.  (The kernels using these do not otherwise use M0.)
template <bool STREAM>
__device__ inline void dma_16s(const void *sbase, uint32_t voff, uint32_t lds_base)
{
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 sc0 nt" ::"v"(voff),
                     "s"(sbase), "s"(lds_base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                     "s"(lds_base)
                     : "memory", "m0");
}

template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Fused scoring + first top-K level (decode): columns per block and ring depth (5 x 16 KB per block,
// reused by the selection; the scores stay in registers): 80 KB, two blocks per CU.
constexpr int kFusedCols = 8192;
constexpr int kFusedRing = 5;
// The 8-wave form (one block per CU): a 4-deep ring of 4 KB per wave, 128 KB per block.
constexpr int kFusedRing8 = 4;

// Block -> (row, chunk) of the streaming kernels.  Blocks go to the 8 XCDs in turn, in launch order
// (chunk fastest), so chunk c of every row lands on the XCD of c mod 8.  The fused selection passes
// (SELECT) are taken chunk by chunk as the paged ones below: in a ragged batch the chunks past a short
// row's range exit at once, and the chunk-major order puts the busy low chunks of all rows first.  A paged row's chunks can
// differ a lot in work (a recall list that is mostly padding leaves its last chunks empty), so paged
// blocks are taken chunk by chunk instead, all rows of a chunk before the next chunk, with the rows
// rotated by the chunk index: the busy first chunks come first and are spread over every XCD, and
// the chunks of one row still land on different XCDs.
template <int MODE, bool CHUNK_MAJOR = MODE == kModePaged>
__device__ inline void stream_block(int &r, int64_t &chunk)
{
    r = blockIdx.y;
    chunk = blockIdx.x;
    if constexpr (CHUNK_MAJOR) {
        const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        chunk = lin / gridDim.y;
        r = (int)((lin % gridDim.y + chunk) % gridDim.y);
    }
}

// With a compact list of the wanted rows (count on the device) the blocks are taken in that list's order,
// chunk by chunk: block i of the (chunks x n_rows) grid is chunk i / count of list row i % count, so every
// block that has work comes before every block that has none.  Returns false for a block without work.
__device__ inline bool stream_block_listed(const int32_t *row_list, const int32_t *row_count, int &r, int64_t &chunk)
{
    const int64_t cnt = *row_count;
    const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    if (lin >= cnt * (int64_t)gridDim.x)
        return false;
    chunk = lin / cnt;
    r = row_list[lin % cnt];
    return true;
}

// Columns of the chunk [c_first, c_last) that can hold keys: [c_begin, c_end) (empty when
// c_begin >= c_end).  A flat column is a token position, so the chunk is cut to the row's range
// [lo, hi) (its start kept on a 64-column group).  A paged chunk is cut to the slots from the first
// to the last one whose page has keys in [lo, hi) (recall lists end in -1 padding, and pages past
// the middle range come last), so the unused slots of a short row stream nothing.  Every thread of
// the block calls it (paged: two barriers).
template <int MODE>
__device__ inline void chunk_key_range(const ColMap &cm, int64_t c_first, int64_t c_last, int64_t &c_begin,
                                       int64_t &c_end)
{
    c_begin = c_first;
    c_end = c_last;
    if constexpr (MODE == kModeFlat || MODE == kModePageMean) {
        c_begin = max(c_first, cm.lo / 64 * 64);
        c_end = min(c_last, cm.hi);
    } else {
        __shared__ int32_t slot_span[2];
        if (threadIdx.x == 0)
            slot_span[0] = INT32_MAX, slot_span[1] = -1;
        __syncthreads();
        const int32_t s_lo = (int32_t)(c_first / cm.P), s_hi = (int32_t)min<int64_t>((c_last + cm.P - 1) / cm.P, cm.M);
        for (int32_t sl = s_lo + (int32_t)threadIdx.x; sl < s_hi; sl += (int32_t)blockDim.x) {
            const int64_t pg = cm.page_row ? cm.page_row[sl] : -1;
            if (pg >= 0 && pg * cm.P < cm.hi && (pg + 1) * cm.P > cm.lo) {
                atomicMin(&slot_span[0], sl);
                atomicMax(&slot_span[1], sl);
            }
        }
        __syncthreads();
        if (slot_span[1] < 0) {
            c_begin = c_last;  // nothing to score
        } else {
            c_begin = max(c_first, (int64_t)slot_span[0] * cm.P / 64 * 64);
            c_end = min(c_last, ((int64_t)slot_span[1] + 1) * cm.P);
        }
    }
}

// SELECT (flat decode rows): instead of writing its scores, the block keeps them in registers and writes
// its chunk's best k_sel (key desc, position asc) as the first-level candidate list of the top-K
// (sel_key / sel_pos [row][chunk * k_sel ..], key 0 / position -1 padded), so the fp32 scores never go
// to HBM (their write traffic, interleaved with the key stream, slowed the stream by ~15 % at 1M).
// LDS words of the fused epilogue for C-column chunks: the selection's histograms and scratch, or the
// emit's (group, wave) counts, scan scratch and staged list (at most min(kMaxLocalK, C) picks).
constexpr int fused_emit_words(int C) { return 2 * (C / kWave) + 16 + 2 * (C < kMaxLocalK ? C : kMaxLocalK); }
constexpr int fused_lds_words(int C)
{
    return kLdsWords + 3 * 16 + 3 > fused_emit_words(C) ? kLdsWords + 3 * 16 + 3 : fused_emit_words(C);
}

// Order key of a score for the selection (0: not a candidate).
__device__ __attribute__((always_inline)) inline uint32_t select_key(float v) { return candidate_key(v); }

// v_mbcnt: the set bits of mask in the lanes below this one.
__device__ __attribute__((always_inline)) inline uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Epilogue of the fused scoring kernels, on keys held in registers (built while the chunk streams, with
// their statistics st): thread (wave w, lane (g, n)) holds in key[j] the order key of the score of
// column (tile0 + 4 (W j + w) + g) * 16 + n (W waves), i.e. of its j-th group of four tiles (0 where
// that column holds no key or lies past the chunk's key range).  Selects the k_sel best under
// (score desc, position asc) with the block radix select, then writes them in position order.  For a
// fixed j, wave w's 64 lanes hold 64 consecutive columns, lane order being column order, and those runs
// follow one another in (j, w) order: so ballots count the picks of each (j, w), a block scan over the
// counts in that order gives each run its first slot, and a lane adds the picks of the lanes below it.
// Ties at the threshold (rare: only when the k-th key's value repeats past k) are ranked the same way,
// in a second count.  The picks are staged in LDS at their slots and the list goes out in coalesced
// stores: the pairs (order key, position) at chunk * k_sel of row r's candidate list, padded with
// (0, -1).  lds: the block's idle ring, fused_lds_words(C) words.
template <int C, int NT = 256>
__device__ inline void fused_select_regs(const uint32_t (&key)[C / NT], KeyStats st, uint32_t *lds, int64_t tile0,
                                         int wave, int r, int64_t chunk, int k_sel, uint32_t *__restrict__ sel_key,
                                         int32_t *__restrict__ sel_pos, int64_t sel_ld)
{
    constexpr int kFusedV = C / NT;      // keys per thread
    constexpr int kWaves = NT / kWave;
    constexpr int kE = kFusedV * kWaves;  // (group, wave) runs of 64 columns
    constexpr int kStage = C < kMaxLocalK ? C : kMaxLocalK;
    static_assert(2 * kWaves <= 16 && kFusedV <= kWave && kE <= NT && C % NT == 0,
                  "a lane per group's count; a thread per run in the scan");
    __syncthreads();  // every wave's ring DMA has landed: the ring's LDS is free
    uint32_t *scratch = lds + kLdsWords;  // 3 words per wave for the block reductions, then 3 more
    int *s_d = reinterpret_cast<int *>(scratch + 3 * kWaves);
    uint32_t *s_above = scratch + 3 * kWaves + 1, *s_bin = scratch + 3 * kWaves + 2;
    const Selection sel = block_select<NT, kFusedV>(key, (uint32_t)k_sel, st, lds, scratch, s_d, s_above, s_bin);
    // picked when x >= t_gt; a tie when x == t_eq (the first sel.k_rem ties in position order)
    const uint32_t t_gt = sel.t_gt, t_eq = sel.t_eq;
    const bool ties = t_eq != 0xffffffffu;  // (uniform)
    uint32_t *cnt = lds, *scan = lds + 2 * kE, *stage_key = scan + 16, *stage_pos = stage_key + kStage;
    const int lane = lane_id();
    const uint32_t pos0 = (uint32_t)(tile0 * kTile) + 64u * (uint32_t)wave + (uint32_t)lane;  // column of key[0]
    // picks (cg) and ties (ce) of run (m, wave), held by lane m
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int m = 0; m < kFusedV; ++m) {
        // (the empty asm ties key m to the counts so far: otherwise the compiler issues all the
        // independent ballots first and holds their masks in scalar registers, which spill)
        uint32_t x = key[m];
        asm volatile("" : "+v"(x), "+v"(cg), "+v"(ce));
        const uint32_t ng = (uint32_t)__popcll(__ballot(x >= t_gt));
        cg = lane == m ? ng : cg;
        if (ties) {
            const uint32_t ne = (uint32_t)__popcll(__ballot(x == t_eq));
            ce = lane == m ? ne : ce;
        }
    }
    __syncthreads();  // the selection's LDS is no longer read
    if (lane < kFusedV)
        cnt[lane * kWaves + wave] = cg, cnt[kE + lane * kWaves + wave] = ce;
    __syncthreads();
    const int t = (int)threadIdx.x;
    const uint32_t rg = t < kE ? cnt[t] : 0u, re = t < kE ? cnt[kE + t] : 0u;
    uint32_t bg, be, tg, te;
    block_scan2<NT>(rg, re, bg, be, tg, te, scan);  // (its barriers order the reads above before the writes)
    if (t < kE)
        cnt[t] = bg, cnt[kE + t] = be;
    __syncthreads();
    uint32_t slot = 0;
    if (!ties) {
#pragma unroll
        for (int m = 0; m < kFusedV; ++m) {
            uint32_t x = key[m];
            asm volatile("" : "+v"(x), "+v"(slot));  // (one ballot at a time, as above)
            const bool gt = x >= t_gt;
            slot = cnt[m * kWaves + wave] + lanes_below(__ballot(gt));
            if (gt) {
                stage_key[slot] = x;
                stage_pos[slot] = pos0 + (uint32_t)(64 * kWaves * m);
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < kFusedV; ++m) {
            uint32_t x = key[m];
            asm volatile("" : "+v"(x), "+v"(slot));  // (as above)
            const bool gt = x >= t_gt, eq = x == t_eq;
            const uint64_t mg = __ballot(gt), me = __ballot(eq);
            const uint32_t e_before = cnt[kE + m * kWaves + wave] + lanes_below(me);
            slot = cnt[m * kWaves + wave] + lanes_below(mg) + (e_before < sel.k_rem ? e_before : sel.k_rem);
            if (gt || (eq && e_before < sel.k_rem)) {
                stage_key[slot] = x;
                stage_pos[slot] = pos0 + (uint32_t)(64 * kWaves * m);
            }
        }
    }
    __syncthreads();
    const uint32_t n_sel = tg + (te < sel.k_rem ? te : sel.k_rem);
    uint32_t *kout = sel_key + (int64_t)r * sel_ld + chunk * k_sel;
    int32_t *pout = sel_pos + (int64_t)r * sel_ld + chunk * k_sel;
    for (uint32_t i = (uint32_t)t; i < (uint32_t)k_sel; i += NT) {
        const bool in = i < n_sel;
        kout[i] = in ? stage_key[i] : 0u;
        pout[i] = in ? (int32_t)stage_pos[i] : -1;
    }
}

template <int MODE, int S, int SEL, int WV = kWavesPerBlock, bool KEEP = false>
__global__ __launch_bounds__(64 * WV) void score_stream_kernel(RowsDev rows, const uint16_t *__restrict__ q_idx,
                                                            const float *__restrict__ w,
                                                            const uint16_t *__restrict__ keys, int k_sink, int k_swa,
                                                            const int32_t *__restrict__ pages, int M, int P,
                                                            const int64_t *__restrict__ sb_off, int B,
                                                            float *__restrict__ scores, int64_t ld, int64_t n_cols,
                                                            int64_t cols_per_block, const uint8_t *row_mode, int want,
                                                            int grouped, int k_sel, uint32_t *__restrict__ sel_key,
                                                            int32_t *__restrict__ sel_pos, int64_t sel_ld,
                                                            const int32_t *row_list, const int32_t *row_count,
                                                            const int32_t *blk_table, const int32_t *blk_count)
{
    static_assert(S >= 2 && 4 * (S - 1) < 64, "ring depth");
    constexpr bool SELECT = SEL > 0;     // SEL: the fused pass's chunk width (0: write the scores)
    constexpr int kThreads = 64 * WV;    // WV waves (the selection runs on all of them)
    constexpr int kFusedV = SELECT ? SEL / kThreads : 1;
    static_assert(!SELECT || (MODE == kModeFlat && S * WV * kTile * kDim * 2 >= 4 * fused_lds_words(SEL)),
                  "the selection reuses the ring for its LDS");
    static_assert(SELECT || WV == kWavesPerBlock, "the scoring form runs 4 waves");
    int r;
    int64_t chunk;
    if (blk_table) {
        // the blocks with work, (row, chunk) in order: block i takes entry i, the rest have none
        const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        if (lin >= *blk_count)
            return;
        r = blk_table[2 * lin];
        chunk = blk_table[2 * lin + 1];
        if (chunk >= (int64_t)gridDim.x)
            return;  // (a row longer than max_kv_len: its lists would not fit the candidate buffers)
    } else if (row_list) {
        if (!stream_block_listed(row_list, row_count, r, chunk))
            return;
    } else {
        stream_block<MODE, MODE == kModePaged || SELECT>(r, chunk);
        if (row_mode && row_mode[r] != want)
            return;
        if (grouped && group_uniform(rows, row_mode, want, r / kGroupRows))
            return;  // scored by the multi-row kernel
    }
    __shared__ __attribute__((aligned(16))) uint16_t ring[S][WV][kTile * kDim];
    const RowInfo ri = row_info(rows, r);
    const SiRanges si = si_ranges(ri, k_sink, k_swa);
    const ColMap cm = make_colmap<MODE>(ri, si, sb_off, pages, r, M, P, B);

    const int lane = lane_id();
    const int n = lane & 15;
    const int g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar tile math
    const int64_t c_first = chunk * cols_per_block;
    if constexpr (SELECT) {
        // chunks past the row's scored range publish no list (fused_row_lists: the later levels read
        // only the lists of the chunks before it), so a short row of a ragged batch costs nothing here
        if (cm.lo >= cm.hi || c_first >= cm.hi)
            return;
    }
    const int64_t c_last = c_first + cols_per_block < n_cols ? c_first + cols_per_block : n_cols;
    float *out = scores + (int64_t)r * ld;
    // Columns of this chunk that can hold keys: [c_begin, c_end); the others are written -inf.
    int64_t c_begin, c_end;
    chunk_key_range<MODE>(cm, c_first, c_last, c_begin, c_end);
    const bool empty = cm.lo >= cm.hi || c_begin >= c_end;  // no keys here (the DMAs need a row of keys)
    if constexpr (MODE == kModePageMean) {
        // Page-mean columns are sub-blocks and the output holds one score per page of G of them (chunks
        // start on whole pages): the pages with no sub-block in [c_begin, c_end) are -inf.
        const int64_t G = cm.G;
        const int64_t p_end = (c_last + G - 1) / G < ld ? (c_last + G - 1) / G : ld;
        const int64_t p_lo = empty ? p_end : c_begin / G, p_hi = empty ? p_end : (c_end + G - 1) / G;
        for (int64_t p = c_first / G + threadIdx.x; p < p_lo; p += blockDim.x)
            out[p] = -INFINITY;
        for (int64_t p = p_hi + threadIdx.x; p < p_end; p += blockDim.x)
            out[p] = -INFINITY;
        if (empty)
            return;
    } else if constexpr (!SELECT) {
        if (empty) {
            for (int64_t c = c_first + threadIdx.x; c < c_last; c += blockDim.x)
                out[c] = -INFINITY;
            return;
        }
        for (int64_t c = c_first + threadIdx.x; c < c_begin; c += blockDim.x)
            out[c] = -INFINITY;
        for (int64_t c = c_end + threadIdx.x; c < c_last; c += blockDim.x)
            out[c] = -INFINITY;
    }
    // SELECT: the order keys of this lane's scores, one per group of four tiles (see fused_select_regs)
    uint32_t skey[kFusedV];
#pragma unroll
    for (int m = 0; m < kFusedV; ++m)
        skey[m] = 0u;
    KeyStats st;
    int64_t sel_tile0 = 0;
    if (!empty) {  // (SELECT: a block without keys still publishes its empty candidate list below)
        u32x4 qa[4][4];
        const uint16_t *qrow = q_idx + (int64_t)r * kHeads * kDim;
    #pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(qrow + (mt * 16 + n) * kDim + g * 8);
    #pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = src[4 * ks];
        }
        float wv[4][4];
    #pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 v = *reinterpret_cast<const f32x4 *>(w + (int64_t)r * kHeads + mt * 16 + 4 * g);
    #pragma unroll
            for (int i = 0; i < 4; ++i)
                wv[mt][i] = v[i];
        }

    #pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
    #pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                loaded_here(qa[mt][ks]);
    #pragma unroll
            for (int i = 0; i < 4; ++i)
                loaded_here(wv[mt][i]);
        }

        // This wave's tiles: groups of 4 consecutive tiles (64 columns) go to the waves in turn, so the
        // block reads one dense window; step k of this wave is tile k % 4 of its group k / 4.  Steps
        // past the wave's K use its last step's tile again (a tile past the chunk, in the last group,
        // re-reads the chunk's last tile).
        constexpr int W = WV;
        const int64_t chunk_tile = c_begin / kTile;
        const int64_t end_tile = (c_end + kTile - 1) / kTile;
        const int64_t n_groups = (end_tile - chunk_tile + 3) / 4;
        const int64_t K = wave < n_groups ? 4 * ((n_groups - wave + W - 1) / W) : 0;
        auto tile_of = [&](int64_t k) __attribute__((always_inline)) -> int64_t {
            return chunk_tile + 4 * ((k >> 2) * W + wave) + (k & 3);
        };
        sel_tile0 = chunk_tile;
        const int64_t safe_key = cm.base + cm.lo;
        const uint32_t ring_base =
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)&ring[0][wave][0];
        constexpr uint32_t kSlotBytes = WV * kTile * kDim * 2;
        // Token position of the first column of a tile (-1: the tile holds no token).  A tile lies in
        // one page (P is a multiple of 16), so the page table is read once per tile, by a scalar load.
        auto tile_pos = [&](int64_t tile) __attribute__((always_inline)) -> int64_t {
            const int64_t c0 = tile * kTile;
            if constexpr (MODE != kModePaged) {
                return c0;
            } else {
                // (columns and slots fit in 32 bits; readfirstlane keeps the index in scalar registers)
                const int slot = __builtin_amdgcn_readfirstlane((int)page_slot(cm, (uint32_t)c0));
                if (slot >= cm.M)
                    return -1;
                const int64_t pg = pages[(int64_t)r * M + slot];
                return pg < 0 ? -1 : pg * cm.P + (c0 - (int64_t)slot * cm.P);
            }
        };
        auto key_of = [&](int64_t tp, int i) __attribute__((always_inline)) -> int64_t {
            const int64_t sp = tp + i;
            return (tp >= 0 && sp >= cm.lo && sp < cm.hi) ? cm.base + sp : -1;
        };
        // A tile is interior when all 16 of its columns hold keys (every tile but those at the ends of
        // the scored range); the DMA, the scoring and the store then need no per-lane checks.
        auto interior = [&](int64_t tp) __attribute__((always_inline)) {
            return tp >= cm.lo && tp + kTile <= cm.hi;
        };
        // DMA instruction j of a tile fills bytes 1024 j .. 1024 j + 1023 of its buffer: key 4 j + g,
        // chunk n ^ (4 j + g); lane_off[j] is that key and chunk's byte offset from the tile's first key.
        uint32_t lane_off[4];
    #pragma unroll
        for (int j = 0; j < 4; ++j)
            lane_off[j] = (uint32_t)((4 * j + g) * kDim * 2 + (n ^ (4 * j + g)) * 16);
        auto issue = [&](int64_t k) __attribute__((always_inline)) {
            const int64_t tile = min(tile_of(k < K ? k : K - 1), end_tile - 1);
            const int64_t tp = tile_pos(tile);
            const uint32_t buf = ring_base + (uint32_t)(k % S) * kSlotBytes;
            if (interior(tp)) {
                const uint16_t *kb = keys + (cm.base + tp) * kDim;
    #pragma unroll
                for (int j = 0; j < 4; ++j)
                    dma_16s<!KEEP>(kb, lane_off[j], buf + j * 1024);
            } else {
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kk = 4 * j + g;
                    const int64_t key = key_of(tp, kk);
                    const int64_t row_k = key >= 0 ? key : safe_key;
                    dma_16<!KEEP>(keys + row_k * kDim + (n ^ kk) * 8, buf + j * 1024);
                }
            }
        };
        // Score of tile k (token position tp of its first column) for key n; every lane group ends with
        // the same 16 values.
        // The tile's operands move from its ring slot to registers first; once those LDS reads are done
        // the slot takes the DMA of tile k + S, so all S slots are in flight during the arithmetic.
        auto score_tile = [&](int64_t k, int64_t tp) __attribute__((always_inline)) -> float {
            wait_vmcnt<4 * (S - 1)>();  // DMA(k) has landed: only DMA(k + 1 .. k + S - 1) may follow it
            const bool any = interior(tp) || __ballot(key_of(tp, n) >= 0) != 0;  // wave-uniform
            u32x4 b[4];
            if (any) {
                const uint16_t *krow = &ring[k % S][wave][n * kDim];
    #pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    b[ks] = *reinterpret_cast<const u32x4 *>(krow + (((4 * ks + g) ^ n) * 8));
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slot k % S is free again
            issue(k + S);
            float v = 0.0f;
            if (any) {
                f32x4 acc[4];
    #pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 bb = __builtin_bit_cast(bf16x8, b[ks]);
    #pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[mt][ks]), bb,
                                                                          acc[mt], 0, 0, 0);
                }
    #pragma unroll
                for (int mt = 0; mt < 4; ++mt)
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v += wv[mt][i] * relu(acc[mt][i]);
            }
            return v;  // this lane group's part (its 16 heads) of key n's score
        };
        // Group k0 / 4 (tiles k0 .. k0 + 3): lane group g takes tile g's 16 scores (-inf past c_end or
        // where a column holds no key), the four tiles' partial scores folded by lane swaps.
        auto group = [&](int64_t k0, int64_t &c) __attribute__((always_inline)) -> float {
            const int64_t tp0 = tile_pos(tile_of(k0)), tp1 = tile_pos(tile_of(k0 + 1));
            const int64_t tp2 = tile_pos(tile_of(k0 + 2)), tp3 = tile_pos(tile_of(k0 + 3));
            const float v0 = score_tile(k0, tp0), v1 = score_tile(k0 + 1, tp1);
            const float v2 = score_tile(k0 + 2, tp2), v3 = score_tile(k0 + 3, tp3);
            const float v = sum_halves32(sum_rows_swap16(v0, v1), sum_rows_swap16(v2, v3));
            const int64_t tp = g == 0 ? tp0 : g == 1 ? tp1 : g == 2 ? tp2 : tp3;
            c = tile_of(k0 + g) * kTile + n;
            return c < c_end && key_of(tp, n) >= 0 ? v : -INFINITY;
        };
        if (K > 0) {
            for (int k = 0; k < S; ++k)
                issue(k);
            if constexpr (SELECT) {
                // The scores stay in registers, as order keys (their conversion and statistics are
                // VALU work the key stream hides): groups in runs of 8 (register indices fixed at
                // compile time), each run copied to its place in skey by a wave-uniform branch.
                for (int64_t j0 = 0; 4 * j0 < K; j0 += 8) {
                    uint32_t part[8];
    #pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        int64_t c;
                        part[jj] = 4 * (j0 + jj) < K ? select_key(group(4 * (j0 + jj), c)) : 0u;
                        st.add(part[jj]);
                    }
    #pragma unroll
                    for (int o = 0; o < kFusedV / 8; ++o)
                        if (j0 == 8 * o) {
    #pragma unroll
                            for (int jj = 0; jj < 8; ++jj)
                                skey[8 * o + jj] = part[jj];
                        }
                }
            } else {
                // Lane group g stores tile g's 16 scores, so one store instruction writes 256 contiguous
                // bytes (whole lines).  The DMA waits above count DMA instructions only: a store between
                // the DMA of a tile and its wait only makes the wait stricter.
                for (int64_t k0 = 0; k0 < K; k0 += 4) {
                    int64_t c;
                    const float v = group(k0, c);
                    if constexpr (MODE == kModePageMean) {
                        // the G sub-blocks of a page are G consecutive lanes of a lane group: their scores
                        // are summed (a sub-block that does not exist adds nothing) and the page's first
                        // lane stores the page score, -inf past the row's last causal page
                        float pv = v == -INFINITY ? 0.0f : v;
                        for (int o = 1; o < cm.G; o <<= 1)
                            pv += __shfl_xor(pv, o, kWave);
                        const int64_t pg = c / cm.G;
                        if (c < c_end && (n & (cm.G - 1)) == 0 && pg < ld)
                            out[pg] = pg <= cm.last_page ? pv : -INFINITY;
                    } else if (c < c_end) {
                        out[c] = v;
                    }
                }
            }
            wait_vmcnt<0>();  // the ring's trailing DMA writes land before the block's LDS is reused
        }
    }
    if constexpr (SELECT)
        fused_select_regs<SEL, kThreads>(skey, st, reinterpret_cast<uint32_t *>(&ring[0][0][0]), sel_tile0, wave, r, chunk,
                                         k_sel, sel_key, sel_pos, sel_ld);
}

// ------------------------------------------------------------------------------------------
// FP8 streaming kernel: the same per-row work with E4M3 codes (128 B per key, one power-of-two scale
// per key and per query head), on the CDNA4 FP8 matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4
// (both operands E4M3, unit block scales).  One 16x16x128 product covers a head block's whole dot
// product, so a 16-key tile takes 4 of them.  Since the key scale is positive,
//     sum_j w_j ReLU(sq_j sk q8_j . k8) = sk * sum_j (w_j sq_j) ReLU(q8_j . k8):
// the query scales fold into the head weights and the key scale multiplies the sum.
//
// A tile (16 keys) arrives by three DMA instructions into a 2304-byte ring slot: two of 1 KB for the
// codes (8 keys each) and one global_load_lds_dword for the 16 key scales (lane l fetches the scale
// of key l % 16, so each is stored four times).  16-byte chunk c of key k sits at chunk slot
// 8 k + (c ^ ((k >> 1) & 7)): the 16 lanes reading chunk c of keys 0..15 hit 16 different 16-byte
// bank groups.  Each step issues exactly 3 DMA instructions, and the waits count them.

// A tile of FP8 keys is half the bytes of a bf16 tile for about the same per-tile instruction work,
// so one wave per SIMD cannot keep enough of them moving: the grid is sized for two blocks per CU
// (decode 32 x 128K: 100 us against 153 us with one), each with a 4-deep ring (37 KB of LDS).
#ifndef LSA_FP8_BLOCKS_PER_CU
#define LSA_FP8_BLOCKS_PER_CU 2
#endif
#ifndef LSA_FP8_RING
#define LSA_FP8_RING 4
#endif
constexpr int kFp8Ring = LSA_FP8_RING;
constexpr int kFp8WideRing = 8;  // the 16384-column fused pass (a 4-deep ring measures the same, 6 slower)
// (the 8-wave form of that pass: 8 x 8 slots of 2304 B, 144 KB, one block per CU)
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
constexpr int kDim8 = 128;                          // bytes per key (E4M3 codes of d_I = 128)
constexpr int kTileCodes8 = kTile * kDim8;          // 2 KB
constexpr int kSlot8 = kTileCodes8 + 64 * 4;        // + the scale copies

// 4 bytes per lane (the key scales), with the cache policy of the key stream they belong to.
template <bool STREAM>
__device__ inline void dma_4s(const void *sbase, uint32_t voff, uint32_t lds_base)
{
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 sc0 nt" ::"v"(voff), "s"(sbase),
                     "s"(lds_base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
                     "s"(lds_base)
                     : "memory", "m0");
}
template <bool STREAM>
__device__ inline void dma_4(const void *src, uint32_t lds_base)
{
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off sc0 nt" ::"v"(src),
                     "s"(lds_base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_base)
                     : "memory", "m0");
}

template <int MODE, int S, int SEL, int WV = kWavesPerBlock, bool KEEP = false>
__global__ __launch_bounds__(64 * WV) void score_fp8_kernel(RowsDev rows, const uint8_t *__restrict__ q8,
                                                         const float *__restrict__ q_scale,
                                                         const float *__restrict__ w, const uint8_t *__restrict__ k8,
                                                         const float *__restrict__ k_scale, int k_sink, int k_swa,
                                                         const int32_t *__restrict__ pages, int M, int P,
                                                         float *__restrict__ scores, int64_t ld, int64_t n_cols,
                                                         int64_t cols_per_block, int k_sel, uint32_t *__restrict__ sel_key,
                                                         int32_t *__restrict__ sel_pos, int64_t sel_ld)
{
    static_assert(S >= 2 && 3 * (S - 1) < 64, "ring depth");
    constexpr bool SELECT = SEL > 0;  // SEL: the fused pass's chunk width (0: write the scores)
    constexpr int kThreads = 64 * WV;  // WV waves (the selection runs on all of them)
    constexpr int kFusedV = SELECT ? SEL / kThreads : 1;
    static_assert(SELECT || WV == kWavesPerBlock, "the scoring form runs 4 waves");
    static_assert(!SELECT || (MODE == kModeFlat && S * WV * kSlot8 >= 4 * fused_lds_words(SEL)),
                  "the selection reuses the ring for its LDS");
    int r;
    int64_t chunk;
    stream_block<MODE, MODE == kModePaged || SELECT>(r, chunk);
    __shared__ __attribute__((aligned(16))) uint8_t ring[S][WV][kSlot8];
    uint32_t skey[kFusedV];  // SELECT: the order keys of this lane's scores, one per group of four tiles
#pragma unroll
    for (int m = 0; m < kFusedV; ++m)
        skey[m] = 0u;
    KeyStats st;
    const RowInfo ri = row_info(rows, r);
    const SiRanges si = si_ranges(ri, k_sink, k_swa);
    const ColMap cm = make_colmap<MODE>(ri, si, nullptr, pages, r, M, P, 1);

    const int lane = lane_id();
    const int n = lane & 15;
    const int g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c_first = chunk * cols_per_block;
    if constexpr (SELECT) {
        if (cm.lo >= cm.hi || c_first >= cm.hi)
            return;  // past the row's scored range: no list (see fused_row_lists)
    }
    const int64_t c_last = c_first + cols_per_block < n_cols ? c_first + cols_per_block : n_cols;
    float *out = scores + (int64_t)r * ld;
    int64_t c_begin, c_end;
    chunk_key_range<MODE>(cm, c_first, c_last, c_begin, c_end);
    const bool empty = cm.lo >= cm.hi || c_begin >= c_end;
    if constexpr (!SELECT) {
        if (empty) {
            for (int64_t c = c_first + threadIdx.x; c < c_last; c += blockDim.x)
                out[c] = -INFINITY;
            return;
        }
        for (int64_t c = c_first + threadIdx.x; c < c_begin; c += blockDim.x)
            out[c] = -INFINITY;
        for (int64_t c = c_end + threadIdx.x; c < c_last; c += blockDim.x)
            out[c] = -INFINITY;
    } else if (empty) {  // no keys here: publish the empty candidate list
        fused_select_regs<SEL, kThreads>(skey, st, reinterpret_cast<uint32_t *>(&ring[0][0][0]), 0, wave, r, chunk, k_sel,
                                         sel_key, sel_pos, sel_ld);
        return;
    }
    // A operand of head block mt: lane (n, g) holds bytes 32 g .. 32 g + 31 of head 16 mt + n; the key
    // operand uses the same byte split, so the product is the full 128-byte dot product.
    i32x8 qa[4];
    const uint8_t *qrow = q8 + (int64_t)r * kHeads * kDim8;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        qa[mt] = *reinterpret_cast<const i32x8 *>(qrow + (mt * 16 + n) * kDim8 + 32 * g);
    float wv[4][4];  // w * q scale of head 16 mt + 4 g + i
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(w + (int64_t)r * kHeads + mt * 16 + 4 * g);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(q_scale + (int64_t)r * kHeads + mt * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wv[mt][i] = a[i] * b[i];
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        loaded_here(qa[mt]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            loaded_here(wv[mt][i]);
    }

    constexpr int W = WV;
    const int64_t chunk_tile = c_begin / kTile;
    const int64_t end_tile = (c_end + kTile - 1) / kTile;
    const int64_t n_groups = (end_tile - chunk_tile + 3) / 4;
    const int64_t K = wave < n_groups ? 4 * ((n_groups - wave + W - 1) / W) : 0;
    auto tile_of = [&](int64_t k) __attribute__((always_inline)) -> int64_t {
        return chunk_tile + 4 * ((k >> 2) * W + wave) + (k & 3);
    };
    const int64_t safe_key = cm.base + cm.lo;
    const uint32_t ring_base =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)&ring[0][wave][0];
    constexpr uint32_t kRingStep = WV * kSlot8;
    auto tile_pos = [&](int64_t tile) __attribute__((always_inline)) -> int64_t {
        const int64_t c0 = tile * kTile;
        if constexpr (MODE == kModeFlat) {
            return c0;
        } else {
            const int slot = __builtin_amdgcn_readfirstlane((int)page_slot(cm, (uint32_t)c0));
            if (slot >= cm.M)
                return -1;
            const int64_t pg = pages[(int64_t)r * M + slot];
            return pg < 0 ? -1 : pg * cm.P + (c0 - (int64_t)slot * cm.P);
        }
    };
    auto key_of = [&](int64_t tp, int i) __attribute__((always_inline)) -> int64_t {
        const int64_t sp = tp + i;
        return (tp >= 0 && sp >= cm.lo && sp < cm.hi) ? cm.base + sp : -1;
    };
    auto interior = [&](int64_t tp) __attribute__((always_inline)) {
        return tp >= cm.lo && tp + kTile <= cm.hi;
    };
    // Code DMA j of a tile: lane l fetches chunk (l % 8) ^ ((k >> 1) & 7) of key k = 8 j + l / 8
    // (byte offset from the tile's first key); the scale DMA: key l % 16.
    uint32_t lane_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int kk = 8 * j + (lane >> 3);
        lane_off[j] = (uint32_t)(kk * kDim8 + (((lane & 7) ^ ((kk >> 1) & 7)) * 16));
    }
    const uint32_t scale_off = (uint32_t)(n * 4);
    auto issue = [&](int64_t k) __attribute__((always_inline)) {
        const int64_t tile = min(tile_of(k < K ? k : K - 1), end_tile - 1);
        const int64_t tp = tile_pos(tile);
        const uint32_t buf = ring_base + (uint32_t)(k % S) * kRingStep;
        if (interior(tp)) {
            const uint8_t *kb = k8 + (cm.base + tp) * kDim8;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                dma_16s<!KEEP>(kb, lane_off[j], buf + j * 1024);
            dma_4s<!KEEP>(k_scale + cm.base + tp, scale_off, buf + kTileCodes8);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kk = 8 * j + (lane >> 3);
                const int64_t key = key_of(tp, kk);
                const int64_t row_k = key >= 0 ? key : safe_key;
                dma_16<!KEEP>(k8 + row_k * kDim8 + (((lane & 7) ^ ((kk >> 1) & 7)) * 16), buf + j * 1024);
            }
            const int64_t key = key_of(tp, n);
            dma_4<!KEEP>(k_scale + (key >= 0 ? key : safe_key), buf + kTileCodes8);
        }
    };
    // this lane group's part (its 16 heads) of key n's unscaled score; sk = the key's scale
    auto score_tile = [&](int64_t k, int64_t tp, float &sk) __attribute__((always_inline)) -> float {
        wait_vmcnt<3 * (S - 1)>();  // DMA(k) has landed: only DMA(k + 1 .. k + S - 1) may follow it
        const bool any = interior(tp) || __ballot(key_of(tp, n) >= 0) != 0;  // wave-uniform
        u32x4 b0 = u32x4{0u, 0u, 0u, 0u}, b1 = b0;
        sk = 0.0f;
        if (any) {
            const uint8_t *slot = &ring[k % S][wave][0];
            const int f = (n >> 1) & 7;
            b0 = *reinterpret_cast<const u32x4 *>(slot + 16 * (8 * n + ((2 * g) ^ f)));
            b1 = *reinterpret_cast<const u32x4 *>(slot + 16 * (8 * n + ((2 * g + 1) ^ f)));
            sk = *reinterpret_cast<const float *>(slot + kTileCodes8 + 4 * n);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slot k % S is free again
        issue(k + S);
        float v = 0.0f;
        if (any) {
            const i32x8 bb = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
            f32x4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], bb, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                           0, 0, 0, 127, 0, 127);
            // acc[mt][i] = q8(head 16 mt + 4 g + i) . k8(key n)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v += wv[mt][i] * relu(acc[mt][i]);
        }
        return v;
    };
    // Group k0 / 4 (tiles k0 .. k0 + 3): lane group g takes tile g's 16 scores (-inf past c_end or
    // where a column holds no key), the four tiles' partial sums folded by lane swaps, then scaled.
    auto group = [&](int64_t k0, int64_t &c) __attribute__((always_inline)) -> float {
        const int64_t tp0 = tile_pos(tile_of(k0)), tp1 = tile_pos(tile_of(k0 + 1));
        const int64_t tp2 = tile_pos(tile_of(k0 + 2)), tp3 = tile_pos(tile_of(k0 + 3));
        float s0, s1, s2, s3;
        const float v0 = score_tile(k0, tp0, s0), v1 = score_tile(k0 + 1, tp1, s1);
        const float v2 = score_tile(k0 + 2, tp2, s2), v3 = score_tile(k0 + 3, tp3, s3);
        const float sk = g == 0 ? s0 : g == 1 ? s1 : g == 2 ? s2 : s3;
        const float v = sum_halves32(sum_rows_swap16(v0, v1), sum_rows_swap16(v2, v3)) * sk;
        const int64_t tp = g == 0 ? tp0 : g == 1 ? tp1 : g == 2 ? tp2 : tp3;
        c = tile_of(k0 + g) * kTile + n;
        return c < c_end && key_of(tp, n) >= 0 ? v : -INFINITY;
    };
    if (K > 0) {
        for (int k = 0; k < S; ++k)
            issue(k);
        if constexpr (SELECT) {
            // The scores stay in registers as order keys (as in the bf16 fused kernel).
            for (int64_t j0 = 0; 4 * j0 < K; j0 += 8) {
                uint32_t part[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    int64_t c;
                    part[jj] = 4 * (j0 + jj) < K ? select_key(group(4 * (j0 + jj), c)) : 0u;
                    st.add(part[jj]);
                }
#pragma unroll
                for (int o = 0; o < kFusedV / 8; ++o)
                    if (j0 == 8 * o) {
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            skey[8 * o + jj] = part[jj];
                    }
            }
        } else {
            for (int64_t k0 = 0; k0 < K; k0 += 4) {
                int64_t c;
                const float v = group(k0, c);
                if (c < c_end)
                    out[c] = v;
            }
        }
        wait_vmcnt<0>();
    }
    if constexpr (SELECT)
        fused_select_regs<SEL, kThreads>(skey, st, reinterpret_cast<uint32_t *>(&ring[0][0][0]), chunk_tile, wave, r, chunk,
                                         k_sel, sel_key, sel_pos, sel_ld);
}

// (explicit instantiations: without them the host stub of the flat kernel is not emitted)
#define LSA_FP8_INSTANCE(MODE, RING, SEL, WV, KEEP)                                                                 \
    template __global__ void score_fp8_kernel<MODE, RING, SEL, WV, KEEP>(                                              \
        RowsDev, const uint8_t *, const float *, const float *, const uint8_t *, const float *, int, int,             \
        const int32_t *, int, int, float *, int64_t, int64_t, int64_t, int, uint32_t *, int32_t *, int64_t);
LSA_FP8_INSTANCE(kModeFlat, kFp8Ring, 0, 4, false)
LSA_FP8_INSTANCE(kModePaged, kFp8Ring, 0, 4, false)
LSA_FP8_INSTANCE(kModePaged, kFp8Ring, 0, 4, true)
LSA_FP8_INSTANCE(kModeFlat, kFp8Ring, kFusedCols, 4, false)
LSA_FP8_INSTANCE(kModeFlat, kFp8WideRing, 2 * kFusedCols, 4, false)
LSA_FP8_INSTANCE(kModeFlat, kFp8WideRing, 2 * kFusedCols, 8, false)
#undef LSA_FP8_INSTANCE

// ------------------------------------------------------------------------------------------
// Multi-row bf16 kernel (prefill): the 16 rows of a group share every key tile, so the keys are read
// from HBM once per group instead of once per row and the work becomes matrix-core bound.
//
// Block = 16 waves, one row each (its 64x128 query block in VGPRs): four waves per SIMD at 128
// registers, so one wave's ReLU / weight epilogue runs beside another's matrix products.  Keys arrive
// in stages of 256 (64 KB) by LDS DMA, double-buffered, one barrier per stage (256 rather than 128
// keys: half the barriers, 1 % faster).  Inside a stage the 16-byte chunk c of key k is stored at slot
// 16 k + (c ^ (k % 16)), so the 16 lanes that read one MFMA operand hit 16 different bank groups.  Four
// tiles are scored before their results are stored: lane group g stores tile g, so one store
// instruction writes 256 contiguous bytes.  Each lane group holds a partial score (its 16 heads) of each
// tile; the four partials are folded by two lane swaps of row pairs and one of halves (six instructions
// for four tiles instead of a full four-step reduction per tile and a select: the epilogue's vector
// instructions share the issue port with the products, 3 % faster).

constexpr int kGroupWaves = 16;
constexpr int kGroupThreads = kGroupWaves * kWave;
constexpr int kStageKeys = 256;
constexpr int kStageTiles = kStageKeys / kTile;              // 16
constexpr int kStageElems = kStageKeys * kDim;               // bf16 elements per stage (64 KB)
constexpr int kStageDma = kStageElems * 2 / (16 * kWave);    // 64 wave-wide 1 KB DMA writes
constexpr int kMinGroupedRows = 64;                          // fewer rows: the per-row kernel only
static_assert(kGroupWaves == kGroupRows, "one row per wave");

template <int MODE>
__global__ __launch_bounds__(kGroupThreads, 1) void score_rows_kernel(
    RowsDev rows, const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const uint16_t *__restrict__ keys,
    int k_sink, int k_swa, const int64_t *__restrict__ sb_off, int P, int G, float *__restrict__ scores, int64_t ld,
    int64_t n_cols, int64_t cols_per_block, const uint8_t *row_mode, int want)
{
    // MODE Flat: columns are token positions, keys are k_idx rows.  MODE PageMean (HI stage 1):
    // columns are sub-blocks, keys their means (k_mean rows from sb_off), and the scores of the G
    // sub-blocks of a page are summed into one page score.
    static_assert(MODE == kModeFlat || MODE == kModePageMean, "flat or page-mean columns");
    const int chunk = blockIdx.x, grp = blockIdx.y;
    if (!group_uniform(rows, row_mode, want, grp))
        return;  // the per-row kernel scores these rows
    // Two stage buffers as distinct objects: the compiler then knows that a DMA into one does not
    // write what is being read from the other, and does not wait for it before those reads.
    __shared__ __attribute__((aligned(16))) uint16_t stage0[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t stage1[kStageElems];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = lane_id();
    const int n = lane & 15;
    const int g = lane >> 4;
    const int r = grp * kGroupRows + wave;

    // Column ranges (columns are below 2^31): every valid row scores [lo, hi_r) -- flat: from k_sink to
    // the end of its mid region cut at L; page-mean: the sub-blocks of its causal pages -- and lanes
    // 0..15 of every wave take one row each and reduce.
    const int32_t gseq = group_seq(rows, grp);  // (-1: no row scores anything, every column is -inf)
    int L = 0;         // keys of the sequence
    int64_t base = 0;
    if (gseq >= 0) {
        base = rows.kv_off[gseq];
        L = (int)(rows.kv_off[gseq + 1] - base);
        if constexpr (MODE == kModePageMean) {
            base = sb_off[gseq];
            L = (int)(sb_off[gseq + 1] - base);
        }
    }
    const int n_keys = L;
    auto last_page = [&](const RowInfo &ri) {  // causal pages p <= floor(t / P) that exist
        return (int)(min(ri.t, ri.L - 1) / P);
    };
    auto row_hi = [&](int rr) {
        const RowInfo ri = row_info(rows, rr);
        if constexpr (MODE == kModePageMean) {
            return ri.valid ? min(n_keys, (last_page(ri) + 1) * G) : 0;
        } else {
            const SiRanges gi = si_ranges(ri, k_sink, k_swa);
            return (int)(gi.mid_hi < ri.L ? gi.mid_hi : ri.L);
        }
    };
    const int lo = MODE == kModePageMean ? 0 : k_sink;
    const int my_hi = row_hi(r);
    int u_hi = row_hi(grp * kGroupRows + n);
    for (int o = 1; o < 16; o <<= 1)
        u_hi = max(u_hi, __shfl_xor(u_hi, o, kWave));
    const int c_begin = chunk * (int)cols_per_block;
    const int c_end = (int)min((int64_t)c_begin + cols_per_block, n_cols);
    int st_first = 0, st_end = 0;  // stages of kStageKeys columns from c_begin that hold scores
    {
        const int a = max(lo, c_begin), b = min(u_hi, c_end);
        if (a < b) {
            st_first = (a - c_begin) / kStageKeys;
            st_end = (b - c_begin + kStageKeys - 1) / kStageKeys;
        }
    }
    const int cmp_lo = c_begin + st_first * kStageKeys;
    const int cmp_hi = min(c_begin + st_end * kStageKeys, c_end);

    // Columns outside the computed stages hold no score for any row of the group.  (Page-mean: the
    // stage and chunk bounds are multiples of G, so these are whole pages.)
    {
        float *o = scores + (int64_t)r * ld;
        const int gc = MODE == kModePageMean ? G : 1;
        for (int64_t c = c_begin / gc + lane; c < cmp_lo / gc; c += kWave)
            o[c] = -INFINITY;
        for (int64_t c = cmp_hi / gc + lane; c < (c_end + gc - 1) / gc && c < ld; c += kWave)
            o[c] = -INFINITY;
    }

    if (st_first < st_end) {
        // A operands of the row, and the head weights of the 16 heads each lane ends up holding.
        u32x4 qa[4][4];
        float wv[4][4];
        {
            const uint16_t *qrow = q_idx + (int64_t)r * kHeads * kDim;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(qrow + (mt * 16 + n) * kDim + g * 8);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    qa[mt][ks] = src[4 * ks];
                f32x4 v = *reinterpret_cast<const f32x4 *>(w + (int64_t)r * kHeads + mt * 16 + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wv[mt][i] = v[i];
            }
        }
        // DMA j = wave + 16 jj of a stage fills slots 64 j .. 64 j + 63, i.e. keys 4 j .. 4 j + 3: this
        // lane moves chunk c16 of key 4 wave + 64 jj + g (the same chunk for every jj).
        const int kk0 = 4 * wave + g;
        const int c16 = n ^ (kk0 & 15);
        const uint16_t *kseq = keys + base * kDim;
        const RowInfo my_ri = row_info(rows, r);
        const int my_last_page = MODE == kModePageMean && my_ri.valid ? last_page(my_ri) : -1;  // -1: empty row
        auto issue_stage = [&](int st, uint16_t *buf) __attribute__((always_inline)) {
            const int col0 = c_begin + st * kStageKeys;
            const uint16_t *ks0 = kseq + (int64_t)col0 * kDim;
            const int lim = L - 1 - col0;  // keys past the sequence re-read its last key
#pragma unroll
            for (int jj = 0; jj < kStageDma / kGroupWaves; ++jj) {
                const int kk = min(kk0 + 64 * jj, lim);
                __builtin_amdgcn_global_load_lds((glb_void *)(ks0 + kk * kDim + c16 * 8),
                                                 (lds_void *)(buf + (wave + kGroupWaves * jj) * kWave * 8), 16, 0, 0);
            }
        };
        float *out = scores + (int64_t)r * ld;

        // Score of tile tt of a stage for key n (every lane group ends with the same value).
        auto score_tile = [&](const uint16_t *buf, int tt) __attribute__((always_inline)) -> float {
            u32x4 b[4];
            const uint16_t *krow = buf + (tt * kTile + n) * kDim;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                b[ks] = *reinterpret_cast<const u32x4 *>(krow + (((4 * ks + g) ^ n) * 8));
            f32x4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 bb = __builtin_bit_cast(bf16x8, b[ks]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[mt][ks]), bb,
                                                                      acc[mt], 0, 0, 0);
            }
            float v = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v += wv[mt][i] * relu(acc[mt][i]);
            return v;
        };

        // One stage: wait for its DMA, start the next stage's into the other buffer, score 8 tiles.
        // Page-mean: the G sub-block scores of a page (G consecutive lanes of a lane group; G is a
        // power of two up to 16) are summed, a sub-block past the sequence adding nothing, and lane
        // n % G == 0 stores the page score, -inf for pages after the row's last causal page.
        auto run_stage = [&](int st, const uint16_t *buf, uint16_t *next) __attribute__((always_inline)) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA writes have landed
            __syncthreads();                                  // ... and every other wave's
            if (st + 1 < st_end)
                issue_stage(st + 1, next);
            const int col0 = c_begin + st * kStageKeys;
            const int rel_lo = lo - col0, rel_hi = min(my_hi, c_end) - col0, rel_end = c_end - col0;
#pragma unroll 1
            for (int t4 = 0; t4 < kStageTiles; t4 += 4) {
                // one tile at a time (four in flight would not fit in 128 registers)
                // partial scores of tiles t4 .. t4 + 3 (each lane group holds its 16 heads' part), folded
                // pairwise: lane group g ends with the whole score of tile t4 + g
                float ya = 0.0f, yb = 0.0f;
#pragma unroll 1
                for (int h = 0; h < 2; ++h) {
                    int tt = t4 + 2 * h;
                    const float p0 = score_tile(buf, tt);
                    // the next tile's operand reads wait for this score (one tile in flight)
                    asm volatile("" : "+s"(tt) : "v"(p0));
                    const float p1 = score_tile(buf, tt + 1);
                    yb = sum_rows_swap16(p0, p1);
                    ya = h == 0 ? yb : ya;
                }
                const float v = sum_halves32(ya, yb);
                const int rel = (t4 + g) * kTile + n;
                if constexpr (MODE == kModePageMean) {
                    float pv = col0 + rel < n_keys ? v : 0.0f;
                    for (int o = 1; o < G; o <<= 1)
                        pv += __shfl_xor(pv, o, kWave);
                    const int pg = (col0 + rel) / G;
                    if (rel < rel_end && (n & (G - 1)) == 0 && pg < ld)
                        out[pg] = pg <= my_last_page ? pv : -INFINITY;
                } else {
                    if (rel < rel_end)
                        out[col0 + rel] = rel >= rel_lo && rel < rel_hi ? v : -INFINITY;
                }
            }
        };
        if (st_first & 1)
            issue_stage(st_first, stage1);
        else
            issue_stage(st_first, stage0);
        int st = st_first;
        if (st & 1) {
            run_stage(st, stage1, stage0);
            ++st;
        }
        for (; st < st_end; st += 2) {
            run_stage(st, stage0, stage1);
            if (st + 1 < st_end)
                run_stage(st + 1, stage1, stage0);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Multi-row bf16 kernel over recalled pages (HI stage 2 of a prefill chunk, P = 128).  Each row of a
// group scores only the M pages it recalled, but the rows of a chunk lie in one sequence and their page
// sets overlap heavily, so the per-row kernel reads most pages once per recalling row.  Here a block
// takes a range of kGpPages pages of the sequence and streams, two pages per stage as the flat
// multi-row kernel streams 256 keys, only those pages of the range that some row of the group recalled
// (each once per group); a wave (one row) scores the pages its own row recalled and skips the others,
// so the matrix work is that of the recalled pages alone.  A page's 128 scores go to the row's slot of
// that page: the output keeps the per-row kernel's layout (slot s, offset o at column s P + o), and
// every column gets the same value as there (Eq. 10 inside mid(t), -inf elsewhere).
//
// Columns the stage loop does not produce -- slots whose page is -1, lies outside the sequence or
// holds no token of the row's middle range, columns from M P to ld, every column of an empty row --
// are written -inf by the blocks of the first page range.  A page listed at several slots of a row is
// scored at one of them, and the wave then copies those scores to the others.
constexpr int kGpPages = 256;  // pages per block
constexpr int kGpP = 128;      // page size this kernel takes (a stage holds two pages)
static_assert(2 * kGpP == kStageKeys && kGpPages % kWave == 0, "two pages per stage");

__global__ __launch_bounds__(kGroupThreads, 1) void score_rows_paged_kernel(
    RowsDev rows, const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const uint16_t *__restrict__ keys,
    int k_sink, int k_swa, const int32_t *__restrict__ pages, int M, float *__restrict__ scores, int64_t ld,
    const uint8_t *row_mode, int want)
{
    const int chunk = blockIdx.x, grp = blockIdx.y;
    if (!group_uniform(rows, row_mode, want, grp))
        return;  // the per-row kernel scores these rows
    __shared__ __attribute__((aligned(16))) uint16_t stage0[kStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t stage1[kStageElems];
    __shared__ int32_t slot_of[kGroupRows][kGpPages];  // row's slot of page page0 + i (-1: not recalled)
    __shared__ uint16_t upage[kGpPages];               // recalled pages of the range (from page0), ascending
    __shared__ uint16_t umask[kGpPages];               // the rows that recalled upage[i]
    __shared__ int32_t ucnt[kGpPages / kWave];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = lane_id();
    const int n = lane & 15;
    const int g = lane >> 4;
    const int r = grp * kGroupRows + wave;

    const int32_t gseq = group_seq(rows, grp);  // every row that lies inside its sequence lies in this one
    int64_t base = 0, L = 0;
    if (gseq >= 0) {
        base = rows.kv_off[gseq];
        L = rows.kv_off[gseq + 1] - base;
    }
    const int64_t n_pages = (L + kGpP - 1) / kGpP;
    const int64_t page0 = (int64_t)chunk * kGpPages;
    const int64_t page_end = min(page0 + kGpPages, n_pages);

    const RowInfo ri = row_info(rows, r);
    const SiRanges si = si_ranges(ri, k_sink, k_swa);
    const int64_t lo = si.mid_lo, hi = si.mid_hi < ri.L ? si.mid_hi : ri.L;  // the row's scored tokens
    float *out = scores + (int64_t)r * ld;
    const int32_t *prow = pages + (int64_t)r * M;
    auto eligible = [&](int64_t pg) { return ri.valid && pg >= 0 && pg < n_pages && pg * kGpP < hi && (pg + 1) * kGpP > lo; };

    if (chunk == 0) {
        // -inf for the slots no page range produces, 64 slots at a time; then the columns past M P
        for (int s0 = 0; s0 < M; s0 += kWave) {
            const int s = s0 + lane;
            const int64_t pg = prow[min(s, M - 1)];
            // (pages past the grid's page ranges -- a sequence longer than the stated maximum -- too)
            uint64_t todo = __ballot(s < M && !(eligible(pg) && pg < (int64_t)gridDim.x * kGpPages));
            while (todo) {
                const int b = __ffsll((long long)todo) - 1;
                todo &= todo - 1;
                out[(int64_t)(s0 + b) * kGpP + 2 * lane] = -INFINITY;
                out[(int64_t)(s0 + b) * kGpP + 2 * lane + 1] = -INFINITY;
            }
        }
        for (int64_t c = (int64_t)M * kGpP + lane; c < ld; c += kWave)
            out[c] = -INFINITY;
    }
    if (page0 >= page_end)
        return;  // (no barrier below is reached by any wave of the block)

    for (int i = tid; i < kGroupRows * kGpPages; i += kGroupThreads)
        (&slot_of[0][0])[i] = -1;
    __syncthreads();
    bool dup = false;  // this lane found a page at two slots of its row
    for (int s0 = 0; s0 < M; s0 += kWave) {
        const int s = s0 + lane;
        const int64_t pg = s < M ? prow[s] : -1;
        if (pg >= page0 && pg < page_end && eligible(pg))
            dup |= atomicCAS(&slot_of[wave][pg - page0], -1, s) != -1;
    }
    __syncthreads();
    // The recalled pages of the range in ascending order, with the rows that recalled each.
    uint32_t my_mask = 0;
    uint64_t my_ballot = 0;
    if (wave < kGpPages / kWave) {
        const int i = wave * kWave + lane;
#pragma unroll
        for (int rr = 0; rr < kGroupRows; ++rr)
            my_mask |= (slot_of[rr][i] >= 0 ? 1u : 0u) << rr;
        my_ballot = __ballot(my_mask != 0);
        if (lane == 0)
            ucnt[wave] = __popcll(my_ballot);
    }
    __syncthreads();
    int total = 0, before = 0;
#pragma unroll
    for (int k = 0; k < kGpPages / kWave; ++k) {
        before += k < wave ? ucnt[k] : 0;
        total += ucnt[k];
    }
    if (wave < kGpPages / kWave && my_mask != 0) {
        const int pos = before + (int)lanes_below(my_ballot);
        upage[pos] = (uint16_t)(wave * kWave + lane);
        umask[pos] = (uint16_t)my_mask;
    }
    __syncthreads();
    total = __builtin_amdgcn_readfirstlane(total);
    const int n_st = (total + 1) / 2;  // stages of two recalled pages (the last may hold one)

    // A operands of the row, and the head weights of the 16 heads each lane ends up holding.
    u32x4 qa[4][4];
    float wv[4][4];
    {
        const uint16_t *qrow = q_idx + (int64_t)r * kHeads * kDim;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(qrow + (mt * 16 + n) * kDim + g * 8);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[mt][ks] = src[4 * ks];
            f32x4 v = *reinterpret_cast<const f32x4 *>(w + (int64_t)r * kHeads + mt * 16 + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wv[mt][i] = v[i];
        }
    }
    // DMA j = wave + 16 jj of a stage fills slots 64 j .. 64 j + 63, i.e. keys 4 j .. 4 j + 3 of the stage:
    // this lane moves chunk c16 of stage key 4 wave + 64 jj + g, which lies in the stage's page jj / 2.
    const int kk0 = 4 * wave + g;
    const int c16 = n ^ (kk0 & 15);
    const uint16_t *kseq = keys + base * kDim;
    auto issue_stage = [&](int st, uint16_t *buf) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < kStageDma / kGroupWaves; ++jj) {
            const int ui = min(2 * st + (jj >> 1), total - 1);  // (a stage of one page re-reads it)
            const int64_t tok = min((page0 + upage[ui]) * kGpP + ((kk0 + 64 * jj) & (kGpP - 1)), L - 1);
            __builtin_amdgcn_global_load_lds((glb_void *)(kseq + tok * kDim + c16 * 8),
                                             (lds_void *)(buf + (wave + kGroupWaves * jj) * kWave * 8), 16, 0, 0);
        }
    };
    auto score_tile = [&](const uint16_t *buf, int tt) __attribute__((always_inline)) -> float {
        u32x4 b[4];
        const uint16_t *krow = buf + (tt * kTile + n) * kDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            b[ks] = *reinterpret_cast<const u32x4 *>(krow + (((4 * ks + g) ^ n) * 8));
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 bb = __builtin_bit_cast(bf16x8, b[ks]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[mt][ks]), bb, acc[mt],
                                                                  0, 0, 0);
        }
        float v = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v += wv[mt][i] * relu(acc[mt][i]);
        return v;
    };
    // One stage: wait for its DMA, start the next stage's, then score the stage's pages this row recalled
    // (four tiles at a time, folded as in the flat multi-row kernel: lane group g ends with tile t4 + g).
    auto run_stage = [&](int st, const uint16_t *buf, uint16_t *next) __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA writes have landed
        __syncthreads();                                  // ... and every other wave's
        if (st + 1 < n_st)
            issue_stage(st + 1, next);
#pragma unroll 1
        for (int t4 = 0; t4 < kStageTiles; t4 += 4) {
            const int ui = 2 * st + t4 / 8;
            if (ui >= total)
                break;
            if (!((__builtin_amdgcn_readfirstlane(umask[ui]) >> wave) & 1))
                continue;  // (wave-uniform) the row did not recall this page
            const int64_t pg = page0 + __builtin_amdgcn_readfirstlane(upage[ui]);
            const int slot = __builtin_amdgcn_readfirstlane(slot_of[wave][pg - page0]);
            float ya = 0.0f, yb = 0.0f;
#pragma unroll 1
            for (int h = 0; h < 2; ++h) {
                int tt = t4 + 2 * h;
                const float p0 = score_tile(buf, tt);
                asm volatile("" : "+s"(tt) : "v"(p0));  // one tile in flight (registers)
                const float p1 = score_tile(buf, tt + 1);
                yb = sum_rows_swap16(p0, p1);
                ya = h == 0 ? yb : ya;
            }
            const float v = sum_halves32(ya, yb);
            const int off = ((t4 + g) & 7) * kTile + n;  // token pg P + off
            const int64_t tok = pg * kGpP + off;
            out[(int64_t)slot * kGpP + off] = tok >= lo && tok < hi ? v : -INFINITY;
        }
    };
    if (n_st > 0)
        issue_stage(0, stage0);
    for (int st = 0; st < n_st; st += 2) {
        run_stage(st, stage0, stage1);
        if (st + 1 < n_st)
            run_stage(st + 1, stage1, stage0);
    }

    // Pages listed at several slots of the row: copy the scored slot's columns to the others.
    if (__ballot(dup) != 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this wave's score stores are done
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // and are read back from L2
        for (int s0 = 0; s0 < M; s0 += kWave) {
            const int s = s0 + lane;
            const int64_t pg = s < M ? prow[s] : -1;
            int src = s;
            if (pg >= page0 && pg < page_end && eligible(pg))
                src = slot_of[wave][pg - page0];
            uint64_t todo = __ballot(src != s);
            while (todo) {
                const int b = __ffsll((long long)todo) - 1;
                todo &= todo - 1;
                const int from = __shfl(src, b, kWave);
                const float v0 = out[(int64_t)from * kGpP + 2 * lane], v1 = out[(int64_t)from * kGpP + 2 * lane + 1];
                out[(int64_t)(s0 + b) * kGpP + 2 * lane] = v0;
                out[(int64_t)(s0 + b) * kGpP + 2 * lane + 1] = v1;
            }
        }
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

// ------------------------------------------------------------------------------------------
// FP8 quantizer of the indexer inputs: per vector (a key's d_I dims, or one query head) the scale is
// 2^e with e the smallest integer such that max|x| <= 448 * 2^e (e = 0 for an all-zero vector); each
// element becomes the E4M3 code nearest to x / 2^e, ties to the even code (no saturation is ever
// needed).  The scaling and the rounding are exact power-of-two operations and one round-to-nearest-
// even, so the codes are bit for bit those of the definition.

// E4M3 code of y, |y| <= 448: the grid quantum at |y| is 2^(E-3) for |y| in [2^E, 2^(E+1)), E >= -6,
// and 2^-9 below 2^-6 (subnormals).
__device__ inline uint32_t e4m3_code(float y)
{
    const float a = fabsf(y);
    int ex;
    (void)frexpf(a, &ex);          // a = f 2^ex, f in [0.5, 1)
    int E = max(ex - 1, -6);
    int nn = (int)rintf(ldexpf(a, 3 - E));  // units of the quantum, rounded to even; 0 .. 16
    if (nn >= 16) {                // the rounding carried into the next binade
        E += 1;
        nn >>= 1;
    }
    uint32_t code = nn >= 8 ? (uint32_t)(((E + 7) << 3) | (nn - 8)) : (uint32_t)nn;
    if (signbit(y) && code != 0u)
        code |= 0x80u;
    return code;
}

template <typename T>
__device__ inline float load_as_float(const T *p);
template <>
__device__ inline float load_as_float<float>(const float *p) { return *p; }
template <>
__device__ inline float load_as_float<uint16_t>(const uint16_t *p) { return bf16_bits_to_float(*p); }

// One wave per vector (dim <= 256: element lane + 64 i in the lane's register i).
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T *__restrict__ x, int64_t n_vec, int dim,
                                                            uint8_t *__restrict__ codes, float *__restrict__ scale)
{
    const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (v >= n_vec)
        return;  // wave-uniform
    const int lane = lane_id();
    const T *xv = x + v * dim;
    float e[4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = lane + 64 * i;
        e[i] = idx < dim ? load_as_float<T>(xv + idx) : 0.0f;
        amax = fmaxf(amax, fabsf(e[i]));
    }
    amax = wave_max(amax);
    int ex;
    const float f = frexpf(amax, &ex);  // amax = f 2^ex; 448 = 0.875 2^9
    const int sexp = amax == 0.0f ? 0 : ex - 9 + (f > 0.875f ? 1 : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = lane + 64 * i;
        if (idx < dim)
            codes[v * dim + idx] = (uint8_t)e4m3_code(ldexpf(e[i], -sexp));
    }
    if (lane == 0)
        scale[v] = ldexpf(1.0f, sexp);
}

// ------------------------------------------------------------------------------------------ host

bool index_score_supported(int dtype, int n_heads, int head_dim)
{
    if (dtype == 1)
        return n_heads == kHeads && head_dim == kDim;
    return n_heads >= 1 && n_heads <= kHeads && (head_dim == 64 || head_dim == 128);
}

// Rows of one launch that read the same keys or means: at least two rows per sequence on average (a
// prefill chunk), so the paged and page-mean streams keep the default cache policy.  Under a row gate
// only some rows run (the index owners of an MTP batch: one per sequence), so the streams stay streaming.
static bool rows_share_keys(const RowsDev &rows, const RowGate &gate)
{
    return gate.row_mode == nullptr && (int64_t)rows.n_rows >= 2 * (int64_t)rows.n_seq;
}

// Columns per block of the bf16 kernels: about one block per CU (256 CUs), at most 16384 columns.
struct ScoreGeom {
    int64_t chunk_elems;
    int n_chunks;
};

static ScoreGeom score_geometry(int64_t n_rows, int64_t n_cols, int blocks_per_cu = 1)
{
    int64_t cpb = n_rows * n_cols / (256 * blocks_per_cu);  // large blocks amortise the ring ramp-up and the Q / w loads
    cpb = (cpb + 63) / 64 * 64;
    if (cpb < 256)
        cpb = 256;
    if (cpb > 16384)
        cpb = 16384;
    return ScoreGeom{cpb, (int)((n_cols + cpb - 1) / cpb)};
}

template <int MODE>
static hipError_t launch_mode(int dtype, const RowsDev &rows, int64_t max_len, const void *q_idx, const float *w,
                              const void *keys, int n_heads, int head_dim, int k_sink, int k_swa,
                              const int64_t *sb_off, const int32_t *pages, int M, int P, int B, float *scores,
                              int64_t ld, int64_t n_cols, RowGate gate, hipStream_t stream)
{
    if (rows.n_rows == 0 || n_cols == 0)
        return hipSuccess;
    if (dtype == 1) {
        const ScoreGeom geo = score_geometry(rows.n_rows, n_cols);
        // (paged rows: the multi-row kernel over recalled pages takes pages of 128 tokens, prefill-like
        // batches of at least a group's worth of rows per sequence -- decode batches keep their compact
        // HI row lists -- and recall lists that cover at least a sixth of the sequence: sparser lists
        // leave a group's waves mostly idle on each streamed page and the block bound by its DMA latency.
        // Measured on 2048-row chunks: 4.9 / 6.3 / 8.5 ms at 256K / 512K / 1M tokens against 6.8 / 7.1 /
        // 8.1 ms for the per-row kernel.)
        const bool grouped =
            (MODE == kModeFlat || MODE == kModePageMean ||
             (MODE == kModePaged && P == kGpP && (int64_t)rows.n_rows >= (int64_t)kGroupRows * rows.n_seq &&
              6 * (int64_t)M * P >= max_len)) &&
            rows.n_rows >= kMinGroupedRows;
        // One sequence, whole groups, no gate: every group is uniform, so the per-row launch would only
        // find rows already scored (a prefill chunk: 73,728 blocks returning at once, 0.3 ms).
        const bool all_grouped = grouped && rows.n_seq == 1 && rows.n_rows % kGroupRows == 0 && !gate.row_mode;
        if constexpr (MODE == kModePaged) {
            if (grouped) {
                const int64_t n_pages = (max(max_len, (int64_t)1) + kGpP - 1) / kGpP;
                dim3 ggrid((unsigned)((n_pages + kGpPages - 1) / kGpPages), (unsigned)(rows.n_rows / kGroupRows));
                hipLaunchKernelGGL(score_rows_paged_kernel, ggrid, dim3(kGroupThreads), 0, stream, rows,
                                   (const uint16_t *)q_idx, w, (const uint16_t *)keys, k_sink, k_swa, pages, M, scores,
                                   ld, gate.row_mode, gate.want);
            }
        }
        if constexpr (MODE == kModeFlat || MODE == kModePageMean) {
            if (grouped) {
                dim3 ggrid((unsigned)geo.n_chunks, (unsigned)(rows.n_rows / kGroupRows));
                hipLaunchKernelGGL(score_rows_kernel<MODE>, ggrid, dim3(kGroupThreads), 0, stream, rows,
                                   (const uint16_t *)q_idx, w, (const uint16_t *)keys, k_sink, k_swa, sb_off, P, P / B,
                                   scores, ld, n_cols, geo.chunk_elems, gate.row_mode, gate.want);
            }
        }
        if (all_grouped) {
            // (nothing left for the per-row kernels)
        } else if constexpr (MODE == kModePageMean) {
            // rows scored one by one stream the means through LDS like the flat rows (chunks of whole
            // 64-column groups, so of whole pages)
            const ScoreGeom sgeo = score_geometry(rows.n_rows, n_cols, LSA_SCORE_BLOCKS_PER_CU);
            dim3 grid((unsigned)sgeo.n_chunks, (unsigned)rows.n_rows);
            auto kernel = rows_share_keys(rows, gate) ? score_stream_kernel<MODE, kScoreRing, 0, kWavesPerBlock, true>
                                                      : score_stream_kernel<MODE, kScoreRing, 0, kWavesPerBlock, false>;
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, rows, (const uint16_t *)q_idx, w,
                               (const uint16_t *)keys, k_sink, k_swa, nullptr, 0, P, sb_off, B, scores, ld, n_cols,
                               sgeo.chunk_elems, gate.row_mode, gate.want, grouped ? 1 : 0, 0, nullptr, nullptr, 0,
                               grouped ? nullptr : gate.list, gate.count, nullptr, nullptr);
        } else {
            ScoreGeom sgeo = score_geometry(rows.n_rows, n_cols, LSA_SCORE_BLOCKS_PER_CU);
            if (MODE == kModePaged && (rows.n_rows < kMinGroupedRows || rows.n_rows < kGroupRows * rows.n_seq) &&
                sgeo.chunk_elems > 2048) {
                // decode-like rows, of which only some (those at least hi_min_len long) may run HI: chunks
                // of 2048 columns (16 pages of 128) keep a few HI rows spread over the whole chip
                sgeo = ScoreGeom{2048, (int)((n_cols + 2047) / 2048)};
            }
            dim3 grid((unsigned)sgeo.n_chunks, (unsigned)rows.n_rows);
            auto kernel = score_stream_kernel<MODE, kScoreRing, 0, kWavesPerBlock, false>;
            if constexpr (MODE == kModePaged) {
                if (rows_share_keys(rows, gate))
                    kernel = score_stream_kernel<MODE, kScoreRing, 0, kWavesPerBlock, true>;
            }
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, rows, (const uint16_t *)q_idx, w,
                               (const uint16_t *)keys, k_sink, k_swa, pages, M, P, nullptr, 1, scores, ld, n_cols,
                               sgeo.chunk_elems, gate.row_mode, gate.want, grouped ? 1 : 0, 0, nullptr, nullptr, 0,
                               grouped ? nullptr : gate.list, gate.count, nullptr, nullptr);
        }
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
                              hipStream_t stream)
{
    if (pages)
        return launch_mode<kModePaged>(dtype, rows, max_kv_len, q_idx, w, k_idx, n_heads, head_dim, k_sink, k_swa,
                                       nullptr, pages, M, P, 1, scores, ld, ld, gate, stream);
    return launch_mode<kModeFlat>(dtype, rows, max_kv_len, q_idx, w, k_idx, n_heads, head_dim, k_sink, k_swa, nullptr,
                                  nullptr, 0, 1, 1, scores, ld, ld, gate, stream);
}

hipError_t launch_page_scores(int dtype, const RowsDev &rows, int64_t max_kv_len, const int64_t *sb_off,
                              const void *q_idx, const float *w, const void *k_mean, int n_heads, int head_dim,
                              int P, int B, float *page_scores, int64_t ld_ps, RowGate gate, hipStream_t stream)
{
    const int G = P / B;
    // Sub-block columns: ld_ps pages x G sub-blocks, so every page column is produced by one tile.
    return launch_mode<kModePageMean>(dtype, rows, max_kv_len, q_idx, w, k_mean, n_heads, head_dim, 0, 0, sb_off,
                                      nullptr, 0, P, B, page_scores, ld_ps, ld_ps * G, gate, stream);
}

hipError_t launch_index_score_fp8(const RowsDev &rows, const uint8_t *q8, const float *q_scale, const float *w,
                                  const uint8_t *k8, const float *k_scale, int k_sink, int k_swa,
                                  const int32_t *pages, int M, int P, float *scores, int64_t ld, hipStream_t stream)
{
    if (rows.n_rows == 0 || ld == 0)
        return hipSuccess;
    const ScoreGeom geo = score_geometry(rows.n_rows, ld, LSA_FP8_BLOCKS_PER_CU);
    dim3 grid((unsigned)geo.n_chunks, (unsigned)rows.n_rows);
    if (pages) {
        auto kernel = rows_share_keys(rows, RowGate{nullptr, 0}) ? score_fp8_kernel<kModePaged, kFp8Ring, 0, 4, true>
                                                                 : score_fp8_kernel<kModePaged, kFp8Ring, 0, 4, false>;
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, rows, q8, q_scale, w, k8, k_scale, k_sink, k_swa, pages,
                           M, P, scores, ld, ld, geo.chunk_elems, 0, nullptr, nullptr, (int64_t)0);
    } else
        hipLaunchKernelGGL((score_fp8_kernel<kModeFlat, kFp8Ring, 0>), grid, dim3(256), 0, stream, rows, q8,
                           q_scale, w, k8, k_scale, k_sink, k_swa, pages, M, P, scores, ld, ld, geo.chunk_elems, 0,
                           nullptr, nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_index_select_fused_fp8(const RowsDev &rows, const uint8_t *q8, const float *q_scale, const float *w,
                                         const uint8_t *k8, const float *k_scale, int k_sink, int k_swa,
                                         int64_t n_cols, int64_t cols, int k, uint32_t *sel_key, int32_t *sel_pos,
                                         int64_t sel_ld, hipStream_t stream)
{
    if (rows.n_rows == 0 || n_cols == 0)
        return hipSuccess;
    dim3 grid((unsigned)((n_cols + cols - 1) / cols), (unsigned)rows.n_rows);
    if (cols == 2 * kFusedCols && (int64_t)grid.x * grid.y >= 512)  // two blocks of 4 waves per CU
        hipLaunchKernelGGL((score_fp8_kernel<kModeFlat, kFp8WideRing, 2 * kFusedCols, 4>), grid, dim3(256), 0, stream,
                           rows, q8, q_scale, w, k8, k_scale, k_sink, k_swa, nullptr, 0, 1, nullptr, (int64_t)0, n_cols,
                           cols, k, sel_key, sel_pos, sel_ld);
    else if (cols == 2 * kFusedCols)  // one round of blocks: one block of 8 waves per CU
        hipLaunchKernelGGL((score_fp8_kernel<kModeFlat, kFp8WideRing, 2 * kFusedCols, 8>), grid, dim3(512), 0, stream,
                           rows, q8, q_scale, w, k8, k_scale, k_sink, k_swa, nullptr, 0, 1, nullptr, (int64_t)0, n_cols,
                           cols, k, sel_key, sel_pos, sel_ld);
    else
        hipLaunchKernelGGL((score_fp8_kernel<kModeFlat, kFp8Ring, kFusedCols>), grid, dim3(256), 0, stream, rows, q8,
                           q_scale, w, k8, k_scale, k_sink, k_swa, nullptr, 0, 1, nullptr, (int64_t)0, n_cols,
                           (int64_t)kFusedCols, k, sel_key, sel_pos, sel_ld);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(int dtype, int64_t n_vec, int dim, const void *x, uint8_t *codes, float *scale,
                               hipStream_t stream)
{
    if (n_vec == 0)
        return hipSuccess;
    dim3 grid((unsigned)((n_vec + 3) / 4));
    if (dtype == 1)
        hipLaunchKernelGGL(quantize_fp8_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t *)x, n_vec, dim,
                           codes, scale);
    else
        hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, dim3(256), 0, stream, (const float *)x, n_vec, dim, codes,
                           scale);
    return hipGetLastError();
}

// Rows are scored one by one (and so can take the fused pass) unless they are prefill-like: many rows
// per sequence, which the 16-row grouped kernel scores from shared key stages.
bool index_select_fusable(int dtype, int n_rows, int n_seq, int n_heads, int head_dim, int k)
{
    const bool per_row = n_rows < kMinGroupedRows || (int64_t)n_rows < (int64_t)kGroupRows * n_seq;
    return dtype == 1 && n_heads == kHeads && head_dim == kDim && per_row && k >= 1 && k <= kMaxLocalK;
}

int64_t index_select_fused_segments(int64_t n_cols) { return (n_cols + kFusedCols - 1) / kFusedCols; }

// Chunk width of the bf16 fused pass: 16384 columns once that gives every CU a block (half the blocks,
// so half the per-block q loads, prologues and candidate lists, and half the candidates of the next
// level), else 8192.
int64_t index_select_fused_cols(int64_t n_rows, int64_t n_cols)
{
    // (a batch of more than 64 rows is taken to be ragged: the chunks of its short rows are empty, so
    // n_rows x chunks overstates the work, and the narrower chunks keep two blocks per CU)
    return n_rows < kMinGroupedRows && n_rows * ((n_cols + 2 * kFusedCols - 1) / (2 * kFusedCols)) >= 256
               ? 2 * kFusedCols
               : kFusedCols;
}

// FP8: the same rule (the 16384-column pass also has a one-round, 8-wave form).
int64_t index_select_fused_cols_fp8(int64_t n_rows, int64_t n_cols)
{
    return n_rows < kMinGroupedRows && n_rows * ((n_cols + 2 * kFusedCols - 1) / (2 * kFusedCols)) >= 256
               ? 2 * kFusedCols
               : kFusedCols;
}

hipError_t launch_index_select_fused(const RowsDev &rows, const void *q_idx, const float *w, const void *k_idx,
                                     int k_sink, int k_swa, int64_t n_cols, int64_t cols, int k, uint32_t *sel_key,
                                     int32_t *sel_pos, int64_t sel_ld, RowGate gate, hipStream_t stream)
{
    if (rows.n_rows == 0 || n_cols == 0)
        return hipSuccess;
    dim3 grid((unsigned)((n_cols + cols - 1) / cols), (unsigned)rows.n_rows);
    if (cols == 2 * kFusedCols && (int64_t)grid.x * grid.y >= 512)  // two blocks of 4 waves per CU
        hipLaunchKernelGGL((score_stream_kernel<kModeFlat, kFusedRing, 2 * kFusedCols>), grid, dim3(256), 0, stream,
                           rows, (const uint16_t *)q_idx, w, (const uint16_t *)k_idx, k_sink, k_swa, nullptr, 0, 1,
                           nullptr, 1, nullptr, (int64_t)0, n_cols, cols, gate.row_mode, gate.want, 0, k, sel_key, sel_pos, sel_ld,
                           gate.list, gate.count, gate.table, gate.table_count);
    else if (cols == 2 * kFusedCols)  // one round of blocks: one block of 8 waves per CU
        hipLaunchKernelGGL((score_stream_kernel<kModeFlat, kFusedRing8, 2 * kFusedCols, 8>), grid, dim3(512), 0,
                           stream, rows, (const uint16_t *)q_idx, w, (const uint16_t *)k_idx, k_sink, k_swa, nullptr, 0,
                           1, nullptr, 1, nullptr, (int64_t)0, n_cols, cols, gate.row_mode, gate.want, 0, k, sel_key, sel_pos,
                           sel_ld, gate.list, gate.count, gate.table, gate.table_count);
    else
        hipLaunchKernelGGL((score_stream_kernel<kModeFlat, kFusedRing, kFusedCols>), grid, dim3(256), 0, stream, rows,
                           (const uint16_t *)q_idx, w, (const uint16_t *)k_idx, k_sink, k_swa, nullptr, 0, 1, nullptr,
                           1, nullptr, (int64_t)0, n_cols, (int64_t)kFusedCols, gate.row_mode, gate.want, 0, k, sel_key, sel_pos,
                           sel_ld, gate.list, gate.count, gate.table, gate.table_count);
    return hipGetLastError();
}

}  // namespace lsa
