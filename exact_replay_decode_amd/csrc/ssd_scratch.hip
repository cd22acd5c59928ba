// ssd_scratch.hip -- the library's own decode bookkeeping array, for the
// entry point that allocates nothing (ssd_replay_decode_static).
//
// The replay-decode kernels keep per-slot arrival counters, done counters
// and the ranking of a large batch in an int32 array of 2 * num_slots + 34
// words that is zero between calls (normally the cache's `work` array). For
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation) the array below
// takes its place: a file-scope device array, one per GPU, held until the
// process ends. Host code never uses the array's name as an address: the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept; kernels receive that pointer.
//
// Calls on one GPU share its array: two calls that overlap in time on one
// GPU (different streams without ordering) race on it. Every call leaves
// the array zero; the first call on a device clears it with a fill kernel
// on the caller's stream (a kernel, not a memset node, so that a captured
// graph replays correctly).
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_internal.hpp"

namespace ssd {
namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kScratchWords = 2 * (int64_t)kStaticMaxSlots + 34;

static __device__ __align__(256) int32_t scratch[kScratchWords];

__global__ void k_fill_zero(int32_t *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

std::mutex g_mu;
int32_t *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_work(int32_t **out, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
            return e;
        k_fill_zero<<<dim3(64), dim3(256), 0, stream>>>(static_cast<int32_t *>(p),
                                                         kScratchWords);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        g_ptr[dev] = static_cast<int32_t *>(p);
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace ssd
