// Bandwidth probe for the benchmark: a plain streaming read of a device
// buffer, the measured ceiling that the bench reports next to the HBM peak
// for read-dominated kernels (the replay decode reads ~99 % of its bytes).
// Built into its own library (libssd_probe.so), loaded only by bench.py; it
// is no part of the scan.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// Block b reads 16-byte words [b per, (b + 1) per) of the buffer, four
// loads per thread in flight; the result is folded into a value that is
// stored only if it equals a pattern the data never produce (so the loads
// cannot be removed and nothing is written in practice).
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ p, size_t per,
                                                      uint32_t *sink) {
    const uint4 *q = p + (size_t)blockIdx.x * per;
    uint32_t acc = 0;
    for (size_t i = threadIdx.x; i < per; i += 4 * blockDim.x) {
        const uint4 a = q[i];
        const uint4 b = i + blockDim.x < per ? q[i + blockDim.x] : make_uint4(0, 0, 0, 0);
        const uint4 c = i + 2 * blockDim.x < per ? q[i + 2 * blockDim.x] : make_uint4(0, 0, 0, 0);
        const uint4 d = i + 3 * blockDim.x < per ? q[i + 3 * blockDim.x] : make_uint4(0, 0, 0, 0);
        acc ^= a.x ^ b.y ^ c.z ^ d.w;
    }
    if (acc == 0x9e3779b9u)
        sink[blockIdx.x] = acc;
}

}  // namespace

// Launch one streaming read of `bytes` (a multiple of 16 * blocks) from the
// device buffer p on `stream`; `sink` holds `blocks` uint32 words. Returns
// a hipError_t value (0 on success).
extern "C" int ssd_probe_stream_read(const void *p, size_t bytes, int blocks, uint32_t *sink,
                                     hipStream_t stream) {
    if (!p || !sink || blocks <= 0 || bytes % (16 * (size_t)blocks) != 0)
        return (int)hipErrorInvalidValue;
    k_stream_read<<<dim3(blocks), dim3(256), 0, stream>>>(static_cast<const uint4 *>(p),
                                                          bytes / 16 / blocks, sink);
    return (int)hipGetLastError();
}
