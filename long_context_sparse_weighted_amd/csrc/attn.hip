// attn.hip -- hybrid sparse attention over the MLA latent KV on gfx950.
//
// For query row r at position t:  S = sink(t) u swa(t) u (indexer picks in mid(t))
//   z_s = scale * q_h . kv_s[0:d_qk],  out_h = sum_s softmax(z)_s kv_s[0:d_v],  lse_h = log sum_s e^{z_s}
// ([summary] "DSA Mechanism Formalization": attention over the selected latent rows; [paper] §4.1.1:
// the contiguous sink+window part and the gathered part are processed separately and merged by
// online-softmax rescaling).
//
// The selected set is enumerated as one list: j < n_sink -> s = j; then the window rows (one
// contiguous run); then the compacted indexer picks.  The list is cut into 32-row tiles; the
// contiguous part is read as whole 1,152-byte rows in address order, the gathered part as
// independent rows, both through the same LDS tile.  A row's list can be split over several
// blocks (flash-decoding style); each writes (m, l, unnormalised o) partials that a merge kernel
// combines with the same rescaling rule.
//
// bf16 kernel, 576 / 512 latent: a block holds 128 heads (8 waves x 16 heads).  Per 32-row tile:
//   S^T[32 rows x 16 heads] = K_tile . Q^T       36 x v_mfma_f32_16x16x32_bf16 (Q^T lives in VGPRs)
//   online softmax per head                      a lane owns one head; two xor shuffles
//   O^T[512 x 16 heads] += V^T_tile . P^T        32 x v_mfma_f32_16x16x32_bf16 (128 accumulators)
// P^T comes straight out of the S^T accumulator layout as the B operand.  Tiles are moved by the
// gfx950 global-to-LDS DMA (global_load_lds_dwordx4) into one of two LDS buffers, so the next tile's
// 1,152-byte rows stream in while the current tile is multiplied, without staging registers.  V^T
// is then built from the K tile in LDS (with the row permutation that matches the accumulator
// layout) using 16-byte stores that touch all 32 banks, so every MFMA operand is one 16-byte LDS
// read.
#include "lsa_kernels.hpp"

namespace lsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowsPerTile = 32;
constexpr int kHeadsPerWave = 16;
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kHeadsPerBlock = kHeadsPerWave * kAttnWaves;
constexpr int kMaxSparse = 4096;
constexpr int kKStride = kDqk + 8;         // bf16 elements per LDS K row (1,168 B)
constexpr int kChunksPerRow = kDqk / 8;    // 72 data chunks of 16 B per row
constexpr int kSlotsPerRow = kKStride / 8; // 73 slots per LDS row (one of padding)
constexpr int kDmaInstr = (32 * kSlotsPerRow + 63) / 64;  // 37 wave-wide 1 KB DMA writes per tile
constexpr int kDmaSlots = kDmaInstr * 64;
constexpr int kVtStride = kRowsPerTile + 8; // bf16 elements per LDS V^T row (80 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplitMerge = 64;

// ------------------------------------------------------------------ selected-set enumeration

struct SelList {
    int64_t base;      // first token row of the sequence
    int n_sink;        // j in [0, n_sink): s = j
    int64_t swa_lo;    // j in [n_sink, n_sink + n_swa): s = swa_lo + (j - n_sink)
    int n_swa;
    int n_sparse;      // j beyond: s = sparse[j - n_sink - n_swa]
    int total;
};

// Compacts the usable indexer picks of a row into LDS (ascending input keeps its order):
// an entry is used when it lies in mid(t) and differs from the entry before it.
__device__ inline int compact_picks(const int32_t *pick_row, int k_sparse, const SiRanges &g, int32_t *sparse,
                                    int32_t *scan_tmp)
{
    // Thread t takes entries [t per, t per + per) (per <= kMaxSparse / 256 = 16 for the block sizes
    // used here), read once into registers with the entry before them (for the repeat test).
    constexpr int kMaxPer = kMaxSparse / 256;
    const int nt = blockDim.x;
    const int tid = threadIdx.x;
    const int per = (k_sparse + nt - 1) / nt;
    const int i0 = tid * per;
    int32_t v[kMaxPer];
    bool ok[kMaxPer];
    int32_t prev = (i0 > 0 && i0 <= k_sparse) ? pick_row[i0 - 1] : INT32_MIN;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
        v[j] = (j < per && i0 + j < k_sparse) ? pick_row[i0 + j] : INT32_MIN;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int32_t s = v[j];
        ok[j] = j < per && i0 + j < k_sparse && s >= g.mid_lo && s < g.mid_hi && (i0 + j == 0 || s != prev);
        prev = s;
        cnt += ok[j] ? 1 : 0;
    }
    // Exclusive scan of the per-thread counts: the wave's in registers, then the wave totals.
    const int lane = lane_id(), wave = tid >> 6, n_waves = nt >> 6;
    const int incl = (int)wave_incl_scan((uint32_t)cnt);
    if (lane == kWave - 1)
        scan_tmp[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int i = 0; i < n_waves; ++i) {
        const int x = scan_tmp[i];
        before += i < wave ? x : 0;
        total += x;
    }
    int o = before + incl - cnt;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
        if (ok[j])
            sparse[o++] = v[j];
    __syncthreads();
    return total;
}

__device__ inline SelList make_sel(const RowInfo &ri, const SiRanges &g, int n_sparse)
{
    SelList L;
    L.base = ri.base;
    L.n_sink = (int)g.sink_hi;
    L.swa_lo = g.swa_lo;
    L.n_swa = (int)(g.swa_hi - g.swa_lo);
    L.n_sparse = ri.valid ? n_sparse : 0;
    L.total = ri.valid ? L.n_sink + L.n_swa + L.n_sparse : 0;
    return L;
}

__device__ inline int64_t sel_pos(const SelList &L, const int32_t *sparse, int j)
{
    if (j < L.n_sink)
        return j;
    j -= L.n_sink;
    if (j < L.n_swa)
        return L.swa_lo + j;
    return sparse[j - L.n_swa];
}

// ------------------------------------------------------------------ fp32 VALU kernel

// One block per (row, head); logits in LDS; three passes (logits, max/sum, weighted sum of V).
__global__ __launch_bounds__(256) void attn_valu_kernel(RowsDev rows, const float *__restrict__ q,
                                                         const float *__restrict__ kv, int n_heads, int d_qk, int d_v,
                                                         float scale, int k_sink, int k_swa, int k_sparse,
                                                         const int32_t *__restrict__ idx, const int32_t *idx_row,
                                                         float *__restrict__ out, float *__restrict__ lse)
{
    const int r = blockIdx.x, h = blockIdx.y;
    __shared__ int32_t sparse[kMaxSparse];
    __shared__ int32_t scan_tmp[256 + 1 + 4];
    __shared__ float z[kMaxSparse + 2048 + 64];
    __shared__ float qs[1024];
    __shared__ float red[8];
    const RowInfo ri = row_info(rows, r);
    const SiRanges g = si_ranges(ri, k_sink, k_swa);
    const int ir = idx_row ? idx_row[r] : r;
    const bool ir_ok = ir >= 0 && ir < rows.n_rows;  // an index row outside idx contributes no picks
    int n_sp = compact_picks(idx + (int64_t)(ir_ok ? ir : 0) * k_sparse, ir_ok ? k_sparse : 0, g, sparse, scan_tmp);
    const SelList L = make_sel(ri, g, n_sp);
    const float *qh = q + ((int64_t)r * n_heads + h) * d_qk;
    for (int d = threadIdx.x; d < d_qk; d += blockDim.x)
        qs[d] = qh[d];
    __syncthreads();
    float *oh = out + ((int64_t)r * n_heads + h) * d_v;
    if (L.total == 0) {
        for (int d = threadIdx.x; d < d_v; d += blockDim.x)
            oh[d] = 0.0f;
        if (lse && threadIdx.x == 0)
            lse[(int64_t)r * n_heads + h] = -INFINITY;
        return;
    }
    const int wave = threadIdx.x >> 6, lane = lane_id();
    for (int j = wave; j < L.total; j += blockDim.x / kWave) {
        const float *kr = kv + (L.base + sel_pos(L, sparse, j)) * d_qk;
        float acc = 0.0f;
        for (int d = lane; d < d_qk; d += kWave)
            acc = fmaf(qs[d], kr[d], acc);
        acc = wave_sum(acc);
        if (lane == 0)
            z[j] = acc * scale;
    }
    __syncthreads();
    float m = -INFINITY;
    for (int j = threadIdx.x; j < L.total; j += blockDim.x)
        m = fmaxf(m, z[j]);
    m = wave_max(m);
    if (lane == 0)
        red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.0f;
    for (int j = threadIdx.x; j < L.total; j += blockDim.x) {
        float p = expf(z[j] - m);
        z[j] = p;
        l += p;
    }
    l = wave_sum(l);
    if (lane == 0)
        red[4 + wave] = l;
    __syncthreads();
    l = red[4] + red[5] + red[6] + red[7];
    const float inv = 1.0f / l;
    for (int d = threadIdx.x; d < d_v; d += blockDim.x) {
        float acc = 0.0f;
        for (int j = 0; j < L.total; ++j)
            acc = fmaf(z[j], kv[(L.base + sel_pos(L, sparse, j)) * d_qk + d], acc);
        oh[d] = acc * inv;
    }
    if (lse && threadIdx.x == 0)
        lse[(int64_t)r * n_heads + h] = m + logf(l);
}

// ------------------------------------------------------------------ bf16 matrix-core kernel

// V^T column order that makes the P^T accumulator rows line up with the MFMA K index: the S^T
// accumulator of lane group g holds tile rows 4g + i and 16 + 4g + i (i < 4), which feed K
// indices 8g + i and 8g + 4 + i.  So V^T column c = 8g + 4a + b holds tile row 16a + 4g + b.
__device__ inline int vt_row(int c) { return 16 * ((c >> 2) & 1) + 4 * (c >> 3) + (c & 3); }

struct AttnPartial {
    uint16_t *o;  // [n_rows][n_split][n_heads][kDv] bf16, normalised by the split's own l
    float *m;     // [n_rows][n_split][n_heads] reference max (log2 domain, scale folded in)
    float *l;     // [n_rows][n_split][n_heads] sum of the split's weights against m
};

__global__ __launch_bounds__(kAttnThreads, 1) void attn_mfma_kernel(RowsDev rows, const uint16_t *__restrict__ q,
                                                                     const uint16_t *__restrict__ kv, int n_heads,
                                                                     float scale, int k_sink, int k_swa, int k_sparse,
                                                                     const int32_t *__restrict__ idx,
                                                                     const int32_t *idx_row, int n_split,
                                                                     uint16_t *__restrict__ out,
                                                                     float *__restrict__ lse, AttnPartial part)
{
    const int split = blockIdx.x, r = blockIdx.y;
    const int h_block = blockIdx.z * kHeadsPerBlock;
    // Two K tiles (the next one arrives by DMA while the current one is used), the V^T tile, the
    // compacted picks and the positions of the current tile's rows.  The two K tiles are distinct
    // objects, each named statically below: the compiler can then tell that the DMA into one does
    // not write the other and does not wait for it before reading the current tile.
    __shared__ __attribute__((aligned(16))) uint16_t kt0[kDmaSlots * 8];
    __shared__ __attribute__((aligned(16))) uint16_t kt1[kDmaSlots * 8];
    __shared__ __attribute__((aligned(16))) uint16_t vt[kDv * kVtStride];
    __shared__ int32_t sparse[kMaxSparse];
    __shared__ int32_t scan_tmp[kAttnThreads + 1 + kAttnWaves];
    __shared__ int32_t tile_ok[2][kRowsPerTile];

    const RowInfo ri = row_info(rows, r);
    const SiRanges g = si_ranges(ri, k_sink, k_swa);
    const int ir = idx_row ? idx_row[r] : r;
    const bool ir_ok = ir >= 0 && ir < rows.n_rows;  // an index row outside idx contributes no picks
    const int n_sp = compact_picks(idx + (int64_t)(ir_ok ? ir : 0) * k_sparse, ir_ok ? k_sparse : 0, g, sparse,
                                   scan_tmp);
    const SelList L = make_sel(ri, g, n_sp);

    const int n_tiles = (L.total + kRowsPerTile - 1) / kRowsPerTile;
    const int tiles_per_split = (n_tiles + n_split - 1) / n_split;
    const int tile_lo = split * tiles_per_split;
    int tile_hi = tile_lo + tiles_per_split;
    if (tile_hi > n_tiles)
        tile_hi = n_tiles;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = lane_id();
    const int n = lane & 15;  // head within the wave (B / C column) and A row
    const int gq = lane >> 4; // lane group 0..3
    const int head = h_block + wave * kHeadsPerWave + n;
    const bool head_ok = head < n_heads;

    // Q^T B-operand fragments: head `head`, depth 144 gq + 8 ks .. +8 for ks < 18.
    u32x4 qb[18];
    {
        const uint16_t *qh = q + ((int64_t)r * n_heads + (head_ok ? head : 0)) * kDqk + gq * 144;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks)
            qb[ks] = *reinterpret_cast<const u32x4 *>(qh + 8 * ks);  // a missing head reads head 0, never stored
    }
    f32x4 o[32];  // O^T[dv = 16 mt + 4 gq + i][head n]
#pragma unroll
    for (int mt = 0; mt < 32; ++mt)
        o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // reference max, log2 domain
    float l_run = 0.0f;       // this lane's rows only; the four lane groups are added at the end
    const float zs = scale * kLog2e;

    auto tile_row_pos = [&](int tile, int row) -> int64_t {
        int j = tile * kRowsPerTile + row;
        return j < L.total ? sel_pos(L, sparse, j) : -1;
    };
    // One tile = 32 rows x 73 16-byte slots (72 of data, one of padding against bank conflicts), moved
    // by wave-wide 1 KB DMA writes: slot s of the tile receives chunk s % 73 of tile row s / 73.
    // Padding slots and rows past the end of the list re-read an existing row of the sequence.
    auto issue_tile = [&](int tile, uint16_t *buf) {
        for (int jj = wave; jj < kDmaInstr; jj += kAttnWaves) {
            const int slot = jj * kWave + lane;
            const int row = slot / kSlotsPerRow, chunk = slot % kSlotsPerRow;
            const int64_t pos = row < kRowsPerTile ? tile_row_pos(tile, row) : -1;
            const int64_t grow = L.base + (pos >= 0 ? pos : 0);
            const int cc = chunk < kChunksPerRow ? chunk : kChunksPerRow - 1;
            const uint16_t *src = kv + grow * kDqk + cc * 8;
            __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(buf + jj * kWave * 8), 16, 0, 0);
        }
    };

    auto run_tile = [&](int tile, const uint16_t *ktc, uint16_t *ktn, int32_t *okc) __attribute__((always_inline)) {
        if (tid < kRowsPerTile)
            okc[tid] = tile_row_pos(tile, tid) >= 0 ? 1 : 0;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of the tile has landed
        __syncthreads();                                  // ... and every other wave's
        if (tile + 1 < tile_hi)
            issue_tile(tile + 1, ktn);
        // V^T from the K tile: item (dv, block of 8 V^T columns) gathers 8 rows of one dv column
        // (consecutive lanes read consecutive dv of one row) and stores them as one 16-byte run.
#pragma unroll
        for (int i = 0; i < (kDv * 4) / kAttnThreads; ++i) {
            int item = tid + kAttnThreads * i;
            int dv = item & (kDv - 1), blk = item / kDv;
            uint32_t e[8];
#pragma unroll
            for (int x = 0; x < 8; ++x)
                e[x] = ktc[vt_row(8 * blk + x) * kKStride + dv];
            u32x4 pk;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                pk[x] = e[2 * x] | (e[2 * x + 1] << 16);
            *reinterpret_cast<u32x4 *>(&vt[dv * kVtStride + 8 * blk]) = pk;
        }
        lds_barrier();  // V^T complete (the next tile's DMA keeps running)

        // S^T = K_tile . Q^T; lane (n, gq) ends with rows 4gq + i (sa) and 16 + 4gq + i (sb) of head n.
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const uint16_t *ra = &ktc[n * kKStride + gq * 144];
            const uint16_t *rb = &ktc[(16 + n) * kKStride + gq * 144];
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                u32x4 a0 = *reinterpret_cast<const u32x4 *>(ra + 8 * ks);
                u32x4 a1 = *reinterpret_cast<const u32x4 *>(rb + 8 * ks);
                bf16x8 bq = __builtin_bit_cast(bf16x8, qb[ks]);
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), bq, sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), bq, sb, 0, 0, 0);
                if ((ks & 1) == 1)
                    __builtin_amdgcn_sched_barrier(0);  // keep only a few LDS fragments live
            }
        }
        // Online softmax in the log2 domain.
        float z[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = okc[4 * gq + i] ? sa[i] * zs : -INFINITY;
            z[4 + i] = okc[16 + 4 * gq + i] ? sb[i] * zs : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            tmax = fmaxf(tmax, z[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        // Move the reference max only when it grows by more than 8 (a factor 256): the softmax is
        // unchanged by the choice of reference, so O^T is rescaled only on those rare steps.
        if (tmax > m_run + 8.0f) {
            float alpha = m_run == -INFINITY ? 0.0f : exp2f(m_run - tmax);
            m_run = tmax;
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < 32; ++mt)
                o[mt] *= alpha;
        }
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float pv = m_run == -INFINITY ? 0.0f : exp2f(z[i] - m_run);
            l_run += pv;
            pb[i] = (__bf16)pv;
        }
        // O^T += V^T . P^T  (one K step of 32 tile rows per 16-dv slice)
        {
            const uint16_t *vrow = &vt[n * kVtStride + 8 * gq];
#pragma unroll
            for (int mt = 0; mt < 32; ++mt) {
                u32x4 a = *reinterpret_cast<const u32x4 *>(vrow + mt * 16 * kVtStride);
                o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[mt], 0, 0, 0);
                if ((mt & 3) == 3)
                    __builtin_amdgcn_sched_barrier(0);
            }
        }
    };



    if (tile_lo < tile_hi) {
        if (tile_lo & 1)
            issue_tile(tile_lo, kt1);
        else
            issue_tile(tile_lo, kt0);
    }
    int tile = tile_lo;
    if (tile < tile_hi && (tile & 1)) {
        run_tile(tile, kt1, kt0, tile_ok[1]);
        ++tile;
    }
    for (; tile < tile_hi; tile += 2) {
        run_tile(tile, kt0, kt1, tile_ok[0]);
        if (tile + 1 < tile_hi)
            run_tile(tile + 1, kt1, kt0, tile_ok[1]);
    }

    float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    if (!head_ok)
        return;
    if (n_split == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t *oh = out + ((int64_t)r * n_heads + head) * kDv;
#pragma unroll
        for (int mt = 0; mt < 32; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oh[mt * 16 + 4 * gq + i] = float_to_bf16_bits(o[mt][i] * inv);
        if (lse && gq == 0)
            lse[(int64_t)r * n_heads + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) / kLog2e : -INFINITY;
    } else {
        const int64_t slot = ((int64_t)r * n_split + split) * n_heads + head;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t *oh = part.o + slot * kDv;
#pragma unroll
        for (int mt = 0; mt < 32; ++mt) {
            uint32_t w0 = (uint32_t)float_to_bf16_bits(o[mt][0] * inv) | ((uint32_t)float_to_bf16_bits(o[mt][1] * inv) << 16);
            uint32_t w1 = (uint32_t)float_to_bf16_bits(o[mt][2] * inv) | ((uint32_t)float_to_bf16_bits(o[mt][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(&oh[mt * 16 + 4 * gq]) = make_uint2(w0, w1);
        }
        if (gq == 0) {
            part.m[slot] = m_run;
            part.l[slot] = l_tot;
        }
    }
}

// ------------------------------------------------------------------ bf16 kernel, 128 heads per block
//
// 4 waves (one per SIMD), 128 heads per block.  Per 32-row tile:
//   QK: wave w computes S^T[32 rows x heads 32w .. 32w + 31] = K_tile . Q^T with 36 x
//       v_mfma_f32_32x32x16_bf16 (its Q^T in VGPRs, K from the tile in LDS), applies the softmax
//       weights and writes P (bf16) to LDS as P[head][row];
//   PV: wave w computes O^T[dv 128w .. 128w + 127 x all 128 heads] += V^T . P^T with 32 x
//       v_mfma_f32_32x32x16_bf16 (256 accumulators, in AGPRs); the V^T operands are read straight
//       from the row-major K tile with the CDNA4 LDS transpose load (ds_read_b64_tr_b16) and the
//       P^T operands from LDS.
// Every wave reads the K tile once, the V^T of its 128 value columns and P once: about a third
// of the LDS traffic of splitting the heads alone over the waves, and no V^T copy.
//
// Softmax reference: the softmax does not depend on it, so each head fixes it once, at the max of
// the block's first tile, and the accumulators are never rescaled in the loop.  Later logits may
// exceed it (weights above 1); if one exceeds it by more than 100 (log2 units, far from the fp32 and
// bf16 overflow at 128) the block runs its tiles again with the observed maximum as reference.

constexpr int kW32 = 4;                       // waves per block
constexpr int kT32 = kW32 * kWave;
#ifndef LSA_QK_AHEAD
#define LSA_QK_AHEAD 4
#endif
constexpr int kH32 = 128;                     // heads per block
constexpr int kPStride = kRowsPerTile + 8;    // bf16 per LDS P row (one head): 80 B
constexpr int kDvPerWave = kDv / kW32;        // 128 value columns per wave in PV

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

// 16 bytes per lane from global memory to LDS at lds_base + 16 * lane (lds_base wave-uniform), issued
// as inline asm: the compiler then inserts no waits for it (it cannot tell which LDS reads the DMA may
// overlap and would wait before every read of the other buffer); the kernel waits for it itself.
__device__ inline void dma_row16(const void *src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const uint16_t *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t *)p;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane r names 4 consecutive bf16 at p; lane j
// receives element j % 4 of the values named by lanes j / 4 + 4 i, i = 0 .. 3.
__device__ inline u32x2 lds_read_tr16(const uint16_t *p)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)(__attribute__((address_space(3))) uint16_t *)p);
    return __builtin_bit_cast(u32x2, v);
}

__global__ __launch_bounds__(kT32, 1) void attn_mfma32_kernel(RowsDev rows, const uint16_t *__restrict__ q,
                                                               const uint16_t *__restrict__ kv, int n_heads,
                                                               float scale, int k_sink, int k_swa, int k_sparse,
                                                               const int32_t *__restrict__ idx,
                                                               const int32_t *idx_row, int n_split,
                                                               uint16_t *__restrict__ out, float *__restrict__ lse,
                                                               AttnPartial part)
{
    // Blocks go to the 8 XCDs in turn, in launch order.  When the rows come in multiples of 8, all the
    // splits of a row go to one XCD: its q (147 KB, read by every split) then comes from that XCD's L2
    // after the first split instead of from HBM once per split.
    int split = blockIdx.x, r = blockIdx.y;
    if (gridDim.z == 1 && gridDim.y % 8 == 0) {
        const int id = blockIdx.x + gridDim.x * blockIdx.y;  // launch order
        const int j = id >> 3;
        r = (id & 7) + 8 * (j / (int)gridDim.x);
        split = j % (int)gridDim.x;
    }
    const int h_block = blockIdx.z * kH32;
    // Two K tiles as distinct objects, each named statically below (the DMA into one does not make
    // the compiler wait before reading the other), the P tile, the compacted picks.
    __shared__ __attribute__((aligned(16))) uint16_t kt0[kDmaSlots * 8];
    __shared__ __attribute__((aligned(16))) uint16_t kt1[kDmaSlots * 8];
    __shared__ __attribute__((aligned(16))) uint16_t pt[kH32 * kPStride];
    __shared__ int32_t sparse[kMaxSparse];
    __shared__ int32_t scan_tmp[kT32 + 1 + kW32];
    __shared__ int32_t tpos[2][kRowsPerTile];  // token positions of a tile's rows (-1: past the list)
    __shared__ float head_m[kH32], head_l[kH32];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = lane_id();
    const int n = lane & 31;   // QK: head 32 wave + n (B / C column) and K tile row (A row)
    const int hh = lane >> 5;  // lane half

    // Q^T B operands of the QK head: depth 16 ks + 8 hh .. +8, ks < 36.  Issued first: their latency
    // overlaps the reads of the row descriptor and of the picks below.
    u32x4 qb[36];
    {
        const uint16_t *qh = q + ((int64_t)r * n_heads + h_block + 32 * wave + n) * kDqk + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < 36; ++ks)
            qb[ks] = *reinterpret_cast<const u32x4 *>(qh + 16 * ks);
    }

    const RowInfo ri = row_info(rows, r);
    const SiRanges g = si_ranges(ri, k_sink, k_swa);
    const int ir = idx_row ? idx_row[r] : r;
    const bool ir_ok = ir >= 0 && ir < rows.n_rows;  // an index row outside idx contributes no picks
    const int n_sp = compact_picks(idx + (int64_t)(ir_ok ? ir : 0) * k_sparse, ir_ok ? k_sparse : 0, g, sparse,
                                   scan_tmp);
    const SelList L = make_sel(ri, g, n_sp);

    const int n_tiles = (L.total + kRowsPerTile - 1) / kRowsPerTile;
    const int tiles_per_split = (n_tiles + n_split - 1) / n_split;
    const int tile_lo = split * tiles_per_split;
    const int tile_hi = min(tile_lo + tiles_per_split, n_tiles);

    // Complete the Q loads here: the compiler's own waits for them inside the tile loop would count
    // the tile DMA too and stall on it.
#pragma unroll
    for (int ks = 0; ks < 36; ++ks)
        asm volatile("" ::"v"(qb[ks]));
    f32x16 o[16];  // index 4 mt + nt: O^T[dv 128 wave + 32 mt + 8 (i/4) + 4 hh + i%4][head 32 nt + n]
    float m_ref = -INFINITY, m_obs = -INFINITY;  // QK head, log2 domain, scale folded in
    float l_run = 0.0f;                          // QK head, this lane's rows
    const float zs = scale * kLog2e;

    auto tile_row_pos = [&](int tile, int row) -> int64_t {
        const int j = tile * kRowsPerTile + row;
        return j < L.total ? sel_pos(L, sparse, j) : -1;
    };
    // One tile = 32 rows x 73 16-byte slots (72 of data, one of padding against bank conflicts), moved
    // by wave-wide 1 KB DMA writes: slot s of the tile receives chunk s % 73 of tile row s / 73.
    // The rows' token positions come from the table tp (filled one tile ahead by 32 threads); padding
    // slots and rows past the end of the list re-read an existing row of the sequence.
    const uint16_t *kv_seq = kv + L.base * kDqk;
    auto fill_table = [&](int tile, int32_t *tp) {
        if (tid < kRowsPerTile)
            tp[tid] = (int32_t)tile_row_pos(tile, tid);
    };
    constexpr int kDmaPerWave = (kDmaInstr + kW32 - 1) / kW32;
    // Wave w moves DMA writes w, w + 4, ... of a tile, either back to back or spread over the QK
    // products of the current tile.  lane_v is the lane index through an opaque copy, taken once per
    // tile: the per-lane offsets are then derived anew for each tile instead of being kept live (and
    // spilled) across the tile loop.
    auto opaque_lane = [&]() __attribute__((always_inline)) {
        uint32_t v;
        asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(lane));
        return v;
    };
    auto issue_one = [&](int t, uint16_t *buf, const int32_t *tp) __attribute__((always_inline)) {
        const int jj = wave + kW32 * t;
        if (jj < kDmaInstr) {
            const uint32_t lane_v = opaque_lane();  // keeps this address math next to its DMA
            const uint32_t slot = jj * kWave + lane_v;
            const uint32_t row = (slot * 57457u) >> 22;  // slot / 73, exact for slot < 2368
            const int32_t pos = tp[row < kRowsPerTile ? row : kRowsPerTile - 1];
            const int chunk = (int)(slot - row * kSlotsPerRow);
            const int cc = chunk < kChunksPerRow ? chunk : kChunksPerRow - 1;
            const uint16_t *src = kv_seq + (int64_t)max(pos, 0) * kDqk + cc * 8;
            dma_row16(src, __builtin_amdgcn_readfirstlane(lds_addr(buf + jj * kWave * 8)));
        }
    };
    auto issue_tile = [&](uint16_t *buf, const int32_t *tp) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < kDmaPerWave; ++t)
            issue_one(t, buf, tp);
    };

    // One tile; when MORE, the next tile's DMA writes are interleaved with its products.
    auto tile_body = [&](bool more, int tile, const uint16_t *ktc, uint16_t *ktn, const int32_t *tpn)
                         __attribute__((always_inline)) {
        // Rows past the end of the list occur in the list's last tile only.
        const int n_valid = min(kRowsPerTile, L.total - tile * kRowsPerTile);
        // QK: S^T[row 8 (i/4) + 4 hh + i%4][head n], i < 16.
        f32x16 s = f32x16{};
        {
            const uint16_t *arow = ktc + n * kKStride + 8 * hh;
            // K operands are read LSA_QK_AHEAD products ahead, so the LDS latency overlaps the products
            // (read just before its product, each one waited out a whole LDS round trip: decode
            // 32 x 128K attention 48.5 -> 46 us).
            constexpr int kAhead = LSA_QK_AHEAD;
            u32x4 ka[kAhead + 1];
#pragma unroll
            for (int j = 0; j < kAhead; ++j)
                ka[j] = *reinterpret_cast<const u32x4 *>(arow + 16 * j);
#pragma unroll
            for (int ks = 0; ks < 36; ++ks) {
                if (ks + kAhead < 36)
                    ka[(ks + kAhead) % (kAhead + 1)] = *reinterpret_cast<const u32x4 *>(arow + 16 * (ks + kAhead));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[ks % (kAhead + 1)]),
                                                            __builtin_bit_cast(bf16x8, qb[ks]), s, 0, 0, 0);
                // Each DMA write stalls this wave's instruction issue for ~100+ cycles: writes 0 .. 4 of
                // the next tile are spread over the QK products, 5 .. 9 over the PV products.
                if (ks % 7 == 3 && more)
                    issue_one(ks / 7, ktn, tpn);
            }
        }
        float tmax = -INFINITY;
        if (n_valid == kRowsPerTile) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[i] *= zs;
                tmax = fmaxf(tmax, s[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 8 * (i >> 2) + 4 * hh + (i & 3);
                s[i] = row < n_valid ? s[i] * zs : -INFINITY;
                tmax = fmaxf(tmax, s[i]);
            }
        }
        tmax = max_xor32(tmax);
        if (m_ref == -INFINITY)
            m_ref = tmax;  // the block's first tile (it always holds a row of the list)
        m_obs = fmaxf(m_obs, tmax);
        // P (bf16) to LDS as P[head][row]: lane (n, hh) holds rows 8 a + 4 hh .. +3 for a < 4.
        uint16_t *prow = pt + (32 * wave + n) * kPStride + 4 * hh;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float pv[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                pv[b] = __builtin_amdgcn_exp2f(s[4 * a + b] - m_ref);  // exp2(-inf) = 0; tiny weights flush to 0
                l_run += pv[b];
            }
            *reinterpret_cast<u32x2 *>(prow + 8 * a) = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        }
        lds_barrier();  // P complete (the next tile's DMA keeps running)
        // PV: 4 dv tiles x 4 head tiles x 2 row steps of 16.
        const int j16 = lane & 15, g16 = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 av[4], bv[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                // lane (g16, j16) names rows 16 ks + 8 (g16 / 2) + 4 t + j16 / 4, columns
                // dv0 + 4 (j16 % 4) .. +3: it then holds V[16 ks + 8 hh + 0 .. 7][dv0 + j16], the A
                // operand V^T[dv][row] of its lane.
                const int dv0 = kDvPerWave * wave + 32 * mt + 16 * (g16 & 1);
                const uint16_t *vp = ktc + (16 * ks + 8 * (g16 >> 1) + (j16 >> 2)) * kKStride + dv0 + 4 * (j16 & 3);
                const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 4 * kKStride);
                av[mt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                bv[nt] = *reinterpret_cast<const u32x4 *>(pt + (32 * nt + n) * kPStride + 16 * ks + 8 * hh);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    o[4 * mt + nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, av[mt]), __builtin_bit_cast(bf16x8, bv[nt]), o[4 * mt + nt], 0, 0,
                        0);
                    const int m = 16 * ks + 4 * mt + nt;
                    if (m % 6 == 3 && m / 6 < kDmaPerWave - 5 && more)
                        issue_one(5 + m / 6, ktn, tpn);
                }
        }
    };
    auto run_tile = [&](int tile, const uint16_t *ktc, uint16_t *ktn, int32_t *tpn) __attribute__((always_inline)) {
        const bool more = tile + 1 < tile_hi;
        if (more)
            fill_table(tile + 1, tpn);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of the tile has landed
        __syncthreads();  // ... and every other wave's; PV of the last tile is done; next table written
        tile_body(more, tile, ktc, ktn, tpn);
    };

    for (int sweep = 0; sweep < 2; ++sweep) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            o[i] = f32x16{};
        l_run = 0.0f;
        if (tile_lo < tile_hi) {
            fill_table(tile_lo, tpos[tile_lo & 1]);
            __syncthreads();
            issue_tile((tile_lo & 1) ? kt1 : kt0, tpos[tile_lo & 1]);
        }
        int tile = tile_lo;
        if (tile < tile_hi && (tile & 1)) {
            run_tile(tile, kt1, kt0, tpos[0]);
            ++tile;
        }
        for (; tile < tile_hi; tile += 2) {
            run_tile(tile, kt0, kt1, tpos[1]);
            if (tile + 1 < tile_hi)
                run_tile(tile + 1, kt1, kt0, tpos[0]);
        }
        // Run again only if some head's logits outgrew its reference by the overflow margin.
        if (!__syncthreads_or(m_obs > m_ref + 100.0f))
            break;
        m_ref = m_obs;
    }

    // Per-head reference and sum from the QK waves, for the value columns of every wave.
    const float l_tot = sum_xor32(l_run);
    if (hh == 0) {
        head_m[32 * wave + n] = m_ref;
        head_l[32 * wave + n] = l_tot;
    }
    __syncthreads();
    // O (normalised, bf16) of the block's 128 heads: the final output, or this split's partial.  Each
    // wave stages 32 heads x its 128 value columns in LDS (the first K tile is free now) and writes
    // them back as whole 256-byte runs of head rows.
    uint16_t *dst = n_split == 1 ? out + ((int64_t)r * n_heads + h_block) * kDv
                                 : part.o + (((int64_t)r * n_split + split) * n_heads + h_block) * kDv;
    constexpr int kStg = kDvPerWave + 8;  // bf16 per staged head row (272 B: rows on different banks)
    uint16_t *stg = kt0 + wave * 32 * kStg;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const float lh = head_l[32 * nt + n];
        const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x16 &acc = o[4 * mt + nt];
                *reinterpret_cast<u32x2 *>(stg + n * kStg + 32 * mt + 8 * i4 + 4 * hh) =
                    u32x2{pack_bf16x2(acc[4 * i4] * inv, acc[4 * i4 + 1] * inv),
                          pack_bf16x2(acc[4 * i4 + 2] * inv, acc[4 * i4 + 3] * inv)};
            }
        // The wave reads back only what its own lanes wrote (a wave's LDS operations complete in order).
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int hrow = 4 * it + (lane >> 4), ch = lane & 15;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + hrow * kStg + 8 * ch);
            *reinterpret_cast<u32x4 *>(dst + (int64_t)(32 * nt + hrow) * kDv + kDvPerWave * wave + 8 * ch) = v;
        }
    }
    if (wave == 0 && hh == 0) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int hl = 32 * nt + n, head = h_block + hl;
            const float mh = head_m[hl], lh = head_l[hl];
            if (n_split == 1) {
                if (lse)
                    lse[(int64_t)r * n_heads + head] = lh > 0.0f ? (mh + log2f(lh)) / kLog2e : -INFINITY;
            } else {
                const int64_t slot = ((int64_t)r * n_split + split) * n_heads + head;
                part.m[slot] = mh;
                part.l[slot] = lh;
            }
        }
    }
}

// Combines the split partials of one (row, head) (one wave per head; lane l owns value columns
// 8 l .. 8 l + 7): split s enters with weight l_s 2^(m_s - M), M the largest m_s.
__global__ __launch_bounds__(256) void attn_merge_kernel(int n_heads, int n_split, AttnPartial part,
                                                          uint16_t *__restrict__ out, float *__restrict__ lse)
{
    const int r = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (h >= n_heads)
        return;
    const int lane = lane_id();
    const int64_t slot0 = (int64_t)r * n_split * n_heads + h;  // split s at slot0 + s n_heads
    float ms = -INFINITY, ls = 0.0f;
    if (lane < n_split) {
        ms = part.m[slot0 + (int64_t)lane * n_heads];
        ls = part.l[slot0 + (int64_t)lane * n_heads];
    }
    const float mx = wave_max(ms);
    const float w = ls > 0.0f ? ls * exp2f(ms - mx) : 0.0f;
    const float l = wave_sum(w);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_split; s0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int sp = min(s0 + k, n_split - 1);
            v[k] = *reinterpret_cast<const u32x4 *>(part.o + (slot0 + (int64_t)sp * n_heads) * kDv + 8 * lane);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(s0 + k, kWave - 1)));
            const float wt = s0 + k < n_split ? wk : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += wt * __uint_as_float(v[k][i] << 16);
                acc[2 * i + 1] += wt * __uint_as_float(v[k][i] & 0xffff0000u);
            }
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    *reinterpret_cast<u32x4 *>(out + ((int64_t)r * n_heads + h) * kDv + 8 * lane) =
        u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
              pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    if (lse && lane == 0)
        lse[(int64_t)r * n_heads + h] = l > 0.0f ? (mx + log2f(l)) / kLog2e : -INFINITY;
}

// ------------------------------------------------------------------ host

constexpr int kMaxSplit = kMaxSplitMerge;

// Splits of each row's selected list: the grid runs in rounds of 256 blocks (one per CU), a block costs
// its tiles plus a fixed part (Q load, pick compaction, partial store: about 5 tiles' worth), so the
// split count minimises rounds x (tiles per split + 5), with at least 2 tiles per split.
static int pick_split(int n_rows, int n_heads, int k_total)
{
    // Time model in units of one 32-row tile step of a block (about 2.4-3.2 us): a launch takes
    // rounds x (tiles per split + 5) units (5 for a block's fixed costs: q loads, pick compaction, the
    // first tile's latency, the output stores), and with ns > 1 the merge kernel adds its launch
    // (about 2.5 us) and its traffic (the bf16 partials read and the output written, at about
    // 4.4 TB/s).  Measured: 8 rows take 22 splits of 3 tiles (29.0 us against 30.8 with 13 of 5; 33 of 2
    // need a second round: 43 us), 32 rows 8, 64 rows 4; 192 rows (a ragged batch of drafts) run
    // unsplit, where 4 splits cost 183 + 25 us of merge.
    const int64_t row_blocks = (int64_t)n_rows * ((n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
    const int n_tiles = (k_total + kRowsPerTile - 1) / kRowsPerTile;
    const int max_split = min(kMaxSplit, max(1, n_tiles / 2));
    constexpr double kUnitUs = 2.8;
    int best = 1;
    double best_cost = 1e300;
    for (int ns = 1; ns <= max_split; ++ns) {
        const int64_t rounds = (row_blocks * ns + 255) / 256;
        double cost = (double)(rounds * ((n_tiles + ns - 1) / ns + 5));
        if (ns > 1) {
            const double bytes = (double)n_rows * n_heads * ((double)ns * (kDv * 2 + 8) + kDv * 2);
            cost += (2.5 + bytes / 4.4e6) / kUnitUs;
        }
        if (cost < best_cost) {
            best_cost = cost;
            best = ns;
        }
    }
    return best;
}

size_t attn_workspace_bytes(int dtype, int n_rows, int n_heads, int d_v, int k_total)
{
    if (dtype != 1)
        return 0;
    int ns = pick_split(n_rows, n_heads, k_total);
    if (ns == 1)
        return 0;
    size_t slots = (size_t)n_rows * ns * n_heads;
    return align_up(slots * kDv * sizeof(uint16_t)) + 2 * align_up(slots * sizeof(float));
}

bool attn_supported(int dtype, int n_heads, int d_qk, int d_v, int k_sparse, int k_total)
{
    if (k_sparse > kMaxSparse)
        return false;
    if (dtype == 1)
        return n_heads % kHeadsPerWave == 0 && d_qk == kDqk && d_v == kDv;
    return d_qk <= 1024 && d_v <= d_qk && k_total <= kMaxSparse + 2048 + 64;
}

hipError_t launch_hybrid_attn(int dtype, const RowsDev &rows, const void *q, const void *kv, int n_heads, int d_qk,
                              int d_v, float scale, int k_sink, int k_swa, int k_sparse, const int32_t *idx,
                              const int32_t *idx_row, void *out, float *lse, void *ws, hipStream_t stream)
{
    if (rows.n_rows == 0)
        return hipSuccess;
    if (dtype != 1) {
        hipLaunchKernelGGL(attn_valu_kernel, dim3(rows.n_rows, n_heads), dim3(256), 0, stream, rows, (const float *)q,
                           (const float *)kv, n_heads, d_qk, d_v, scale, k_sink, k_swa, k_sparse, idx, idx_row,
                           (float *)out, lse);
        return hipGetLastError();
    }
    const int k_total = k_sink + k_swa + k_sparse;
    const int ns = pick_split(rows.n_rows, n_heads, k_total);
    AttnPartial part{nullptr, nullptr, nullptr};
    if (ns > 1) {
        size_t slots = (size_t)rows.n_rows * ns * n_heads;
        char *p = (char *)ws;
        part.o = (uint16_t *)p;
        p += align_up(slots * kDv * sizeof(uint16_t));
        part.m = (float *)p;
        p += align_up(slots * sizeof(float));
        part.l = (float *)p;
    }
    dim3 grid(ns, rows.n_rows, (n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
    if (n_heads % kH32 == 0)
        hipLaunchKernelGGL(attn_mfma32_kernel, grid, dim3(kT32), 0, stream, rows, (const uint16_t *)q,
                           (const uint16_t *)kv, n_heads, scale, k_sink, k_swa, k_sparse, idx, idx_row, ns,
                           (uint16_t *)out, lse, part);
    else
        hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(kAttnThreads), 0, stream, rows, (const uint16_t *)q,
                           (const uint16_t *)kv, n_heads, scale, k_sink, k_swa, k_sparse, idx, idx_row, ns,
                           (uint16_t *)out, lse, part);
    if (ns > 1)
        hipLaunchKernelGGL(attn_merge_kernel, dim3(rows.n_rows, (n_heads + 3) / 4), dim3(256), 0, stream, n_heads, ns, part,
                           (uint16_t *)out, lse);
    return hipGetLastError();
}

}  // namespace lsa
