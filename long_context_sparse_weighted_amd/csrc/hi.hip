// hi.hip -- the sub-block mean cache of Hierarchical Indexing ([paper] §3.3 "Design choices": the
// block means are precomputed once per sequence and cached; [review] §2.3).
//
// Sub-block n of sequence b covers tokens [nB, min((n+1)B, L_b)); its mean key is the fp64 sum of
// the tokens present (exact for bf16 and fp32 inputs of ordinary range) divided by their count and
// rounded once to the storage dtype.  One thread per (sub-block, dim): consecutive threads walk
// consecutive dims of the same token rows, so every token row is read as one coalesced run.
#include "lsa_kernels.hpp"

namespace lsa {

template <typename T>
__device__ inline double to_double(T v);
template <>
__device__ inline double to_double<float>(float v) { return (double)v; }
template <>
__device__ inline double to_double<uint16_t>(uint16_t v) { return (double)bf16_bits_to_float(v); }

template <typename T>
__device__ inline T from_double(double v);
template <>
__device__ inline float from_double<float>(double v) { return (float)v; }
template <>
__device__ inline uint16_t from_double<uint16_t>(double v) { return double_to_bf16_bits(v); }

// Sub-blocks rebuilt for sequence b: n_first(b) .. nsb(b) - 1, where n_first is the sub-block of token
// first_token (the whole cache from there on), or, when n_new > 0, that of token L_b - n_new (the
// sequence's n_new newest tokens: the per-step upkeep after appending).  Thread (j, d) of sequence b
// takes sub-block n_first(b) + j.
template <typename T>
__global__ __launch_bounds__(256) void page_means_kernel(const int64_t *kv_off, const int64_t *sb_off,
                                                          const T *__restrict__ k_idx, int head_dim, int B,
                                                          int64_t first_token, int64_t n_new, T *__restrict__ k_mean)
{
    const int b = blockIdx.y;
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int d = (int)(item % head_dim);
    const int64_t base = kv_off[b];
    const int64_t L = kv_off[b + 1] - base;
    const int64_t nsb = (L + B - 1) / B;
    const int64_t first = n_new > 0 ? (L > n_new ? L - n_new : 0) : first_token;
    const int64_t n = first / B + item / head_dim;
    if (n >= nsb)
        return;
    const int64_t lo = n * B;
    int64_t hi = lo + B;
    if (hi > L)
        hi = L;
    double sum = 0.0;
    for (int64_t s = lo; s < hi; ++s)
        sum += to_double<T>(k_idx[(base + s) * head_dim + d]);
    k_mean[(sb_off[b] + n) * head_dim + d] = from_double<T>(sum / (double)(hi - lo));
}

hipError_t launch_page_means(int dtype, int n_seq, const int64_t *kv_off, const int64_t *sb_off, const void *k_idx,
                             int head_dim, int B, int64_t max_kv_len, int64_t first_token, int64_t n_new,
                             void *k_mean, hipStream_t stream)
{
    if (n_seq == 0 || max_kv_len == 0 || (n_new == 0 && first_token >= max_kv_len))
        return hipSuccess;
    // sub-blocks per sequence that can need a rebuild: from the first one touched to the last one
    const int64_t span = n_new > 0 ? (n_new + B - 1) / B + 1 : (max_kv_len + B - 1) / B - first_token / B;
    const int64_t items = span * head_dim;
    dim3 grid((unsigned)((items + 255) / 256), (unsigned)n_seq);
    if (dtype == 1)
        hipLaunchKernelGGL(page_means_kernel<uint16_t>, grid, dim3(256), 0, stream, kv_off, sb_off,
                           (const uint16_t *)k_idx, head_dim, B, first_token, n_new, (uint16_t *)k_mean);
    else
        hipLaunchKernelGGL(page_means_kernel<float>, grid, dim3(256), 0, stream, kv_off, sb_off, (const float *)k_idx,
                           head_dim, B, first_token, n_new, (float *)k_mean);
    return hipGetLastError();
}

}  // namespace lsa
