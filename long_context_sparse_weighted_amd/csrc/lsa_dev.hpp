// lsa_dev.hpp -- device-side helpers shared by the liblsa kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Address spaces of the LDS-DMA builtin's operands.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Rows of a batch as the kernels see them (device pointers).
struct RowsDev {
    const int64_t *kv_off;
    const int32_t *row_seq;
    const int32_t *row_pos;
    int32_t n_rows;
    int32_t n_seq;
};

// Where row r lives: its sequence's first token row, length and position.  A row outside its
// sequence (bad t or bad sequence id) is marked invalid and every range below comes out empty.
struct RowInfo {
    int64_t base;
    int64_t L;
    int64_t t;
    int32_t seq;
    bool valid;
};

__device__ inline RowInfo row_info(const RowsDev &rows, int r)
{
    RowInfo ri;
    int32_t b = rows.row_seq[r];
    ri.seq = b;
    if (b < 0 || b >= rows.n_seq) {
        ri.base = 0, ri.L = 0, ri.t = -1, ri.valid = false;
        return ri;
    }
    ri.base = rows.kv_off[b];
    ri.L = rows.kv_off[b + 1] - ri.base;
    ri.t = rows.row_pos[r];
    ri.valid = ri.t >= 0 && ri.t < ri.L;
    return ri;
}

// The streaming-aware split of the prefix [0, t] into three disjoint half-open ranges:
// sink = the first k_sink tokens, window = the last k_swa tokens (never reaching into the sink),
// mid = what lies between them (the only part the indexer scores).
struct SiRanges {
    int64_t sink_hi;          // sink  = [0, sink_hi)
    int64_t swa_lo, swa_hi;   // window = [swa_lo, swa_hi)
    int64_t mid_lo, mid_hi;   // mid   = [mid_lo, mid_hi)
};

__device__ inline SiRanges si_ranges(const RowInfo &ri, int k_sink, int k_swa)
{
    SiRanges g;
    if (!ri.valid) {
        g.sink_hi = g.swa_lo = g.swa_hi = g.mid_lo = g.mid_hi = 0;
        return g;
    }
    const int64_t t1 = ri.t + 1;
    g.sink_hi = t1 < k_sink ? t1 : (int64_t)k_sink;
    g.swa_hi = t1;
    int64_t lo = t1 - k_swa;
    g.swa_lo = lo < k_sink ? (int64_t)k_sink : lo;
    if (g.swa_lo > t1)
        g.swa_lo = t1;
    g.mid_lo = k_sink;
    g.mid_hi = lo < k_sink ? (int64_t)k_sink : lo;
    return g;
}

// Candidate lists of row r after a fused scoring + first top-K pass on chunks of C columns: one list per
// chunk from column 0 to the end of the row's scored range min(mid_hi, L), none when that range is
// empty.  Chunks past it write nothing, and the later top-K levels read only these lists.
__device__ inline int64_t fused_row_lists(const RowsDev &rows, int r, int k_sink, int k_swa, int64_t C)
{
    const RowInfo ri = row_info(rows, r);
    const SiRanges g = si_ranges(ri, k_sink, k_swa);
    const int64_t hi = g.mid_hi < ri.L ? g.mid_hi : ri.L;
    return hi > g.mid_lo ? (hi + C - 1) / C : 0;
}

// ------------------------------------------------------------------------------- bf16 / floats

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ inline uint16_t float_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp64 -> bf16 bits in one rounding step (nearest even), by integer rounding of the binary64
// significand; values below bf16's normal range round on the fixed 2^-133 subnormal grid.
__device__ inline uint16_t double_to_bf16_bits(double x)
{
    uint64_t bits = (uint64_t)__double_as_longlong(x);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    uint64_t mag = bits & 0x7fffffffffffffffull;
    if (mag >= 0x7ff0000000000000ull)  // inf or NaN
        return mag == 0x7ff0000000000000ull ? (uint16_t)(sign | 0x7f80u) : (uint16_t)0x7fc0u;
    if (mag == 0)
        return sign;
    int e = (int)(mag >> 52) - 1023;      // unbiased exponent (binary64 subnormals land below -126)
    if (e < -126) {
        double scaled = __longlong_as_double((long long)mag) * 0x1p133;  // exact power-of-two scaling
        double r = rint(scaled);                                         // ties to even
        return (uint16_t)(sign | (uint16_t)r);                           // r <= 128: 128 is 2^-126
    }
    uint64_t sig = (mag & 0x000fffffffffffffull) | 0x0010000000000000ull;  // 53-bit significand
    uint64_t keep = sig >> 45;                                             // top 8 bits
    uint64_t rest = sig & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rest > half || (rest == half && (keep & 1)))
        ++keep;
    if (keep == 256) {  // carried into the next binade
        keep = 128;
        ++e;
    }
    if (e > 127)
        return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (uint16_t)((e + 127) << 7) | (uint16_t)(keep & 0x7f));
}

// Order-preserving map of a float onto uint32 (larger float -> larger key); -0 is folded onto +0.
__device__ inline uint32_t float_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A selection candidate is any score that is neither -inf nor NaN.
__device__ inline bool is_candidate(float f)
{
    uint32_t u = __float_as_uint(f);
    return u != 0xff800000u && (u & 0x7fffffffu) <= 0x7f800000u;
}

// is_candidate(f) ? float_order_key(f) : 0 in fewer operations: the map u ^ (sign ? 0xffffffff :
// 0x80000000) sends every candidate to [0x00800000, 0xff800000] (+inf to its top) and -inf and the NaNs
// outside it, and -0 to 0x7fffffff, one below the key of +0, which it takes.
__device__ inline uint32_t candidate_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    k = k == 0x7fffffffu ? 0x80000000u : k;
    return k - 0x00800000u <= 0xff000000u ? k : 0u;
}

// ------------------------------------------------------------------------------- wave helpers

// Workgroup barrier that orders LDS only: this wave's LDS operations complete, then all waves
// meet.  Unlike __syncthreads() it does not wait for outstanding global loads (an LDS DMA in
// flight keeps running); the memory clobber keeps the compiler from moving accesses across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline int lane_id() { return __lane_id(); }

// Cross-lane pair sums on the VALU with the CDNA4 lane swaps (no LDS round trip).
// permlane32_swap(a, b) exchanges the upper 32 lanes of a with the lower 32 lanes of b, so the two
// results add up to a[l] + a[l + 32] in lanes l < 32 and b[l - 32] + b[l] in lanes l >= 32.
// Inclusive prefix sum over the 64 lanes of a wave in registers (DPP): row shifts 1, 2, 4, 8 scan
// each row of 16 lanes, then row broadcasts add lane 15 to rows 1 and 3 and lane 31 to rows 2 and 3.
__device__ inline uint32_t wave_incl_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Lane swaps over lane groups (lane group g = lane / 16).  sum_halves32(a, b): the lower half (groups 0
// and 1) gets a summed over the two 32-lane halves, the upper half gets b summed likewise.
// sum_rows_swap16(a, b): groups 0 and 2 get a summed over their group pair (0+1, 2+3), groups 1 and 3 get
// b (permlane16_swap exchanges the odd 16-lane rows of its first operand with the even rows of its
// second).  So sum_halves32(sum_rows_swap16(p0, p1), sum_rows_swap16(p2, p3)) leaves group g with p_g
// summed over all four groups: six instructions fold four partials.
__device__ inline float sum_halves32(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Every lane: v[l] + v[l ^ 32].
__device__ inline float sum_xor32(float v) { return sum_halves32(v, v); }
__device__ inline float sum_rows_swap16(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline float max_xor32(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ inline float wave_sum(float v)
{
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ inline float wave_max(float v)
{
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

}  // namespace lsa
