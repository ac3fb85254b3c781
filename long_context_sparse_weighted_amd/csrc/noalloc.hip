// noalloc.hip -- lsa_index_topk_noalloc: the flat token selection of lsa_index_topk with its
// workspace in a device array of this library instead of a caller buffer, for callers that may not
// allocate device memory (code under graph capture, serving loops, hosts that forbid it).
//
// The array is a file-scope __device__ variable, so each GPU the library runs on holds its own copy
// from the first call on that GPU until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and is kept per device.
// The kernels write every scratch word they later read within the same call (candidate lists and
// their levels), so nothing has to start at zero and stale contents of an earlier call are never
// read.  Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (two
// streams, or two host threads) race on it and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/lsa.h"
#include "lsa_kernels.hpp"

namespace {

constexpr size_t kScratchBytes = LSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once taken

// The device address of this device's copy of `scratch`.
hipError_t scratch_address(int dev, void **p)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *a = nullptr;
        hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = a;
    }
    *p = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int lsa_index_topk_noalloc(int dtype, const lsa_rows_t *rows, const void *q_idx, const float *w, const void *k_idx,
                           int32_t n_heads, int32_t head_dim, lsa_budget_t budget, int32_t *idx,
                           hipStream_t stream)
{
    // Host-side checks first (no HIP call): the argument checks of lsa_index_topk, then the size.
    size_t need = 0;
    if (int st = lsa::index_topk_check(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, budget, idx, &need))
        return st;
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof msg, "lsa_index_topk_noalloc: these rows need %zu bytes of scratch, more than the %zu "
                 "the library holds; call lsa_index_topk with a workspace", need, kScratchBytes);
        return lsa::set_error(LSA_ERR_UNSUPPORTED, msg);
    }
    if (!rows->n_rows)
        return lsa_index_topk(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, budget, idx, nullptr, 0, stream);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && stream) {
        int sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e == hipSuccess && sdev != dev)
            return lsa::set_error(LSA_ERR_INVALID,
                                  "lsa_index_topk_noalloc: the stream belongs to another device than the current one");
    }
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices))
        return lsa::set_error(LSA_ERR_UNSUPPORTED, "lsa_index_topk_noalloc: device ordinal beyond 63");
    void *ws = nullptr;
    if (e == hipSuccess)
        e = scratch_address(dev, &ws);
    if (e != hipSuccess) {
        char msg[160];
        snprintf(msg, sizeof msg, "lsa_index_topk_noalloc: %s", hipGetErrorString(e));
        return lsa::set_error(LSA_ERR_HIP, msg);
    }
    return lsa_index_topk(dtype, rows, q_idx, w, k_idx, n_heads, head_dim, budget, idx, ws, kScratchBytes, stream);
}

}  // extern "C"
