// Measurement helper for bench.py (not part of the library): the achievable HBM read rate
// for a given byte count, the ceiling a weight-streaming kernel is set beside.
//
// One 256-thread workgroup per quarter CU reads a contiguous share of the buffer with 16-byte
// loads, four in flight per thread, and folds what it read into one word that it stores, so
// that the loads cannot be dropped.  bench_read_launch() takes device pointers and a byte
// count that is a multiple of 16; it launches on the given stream and returns the HIP error
// code of the launch.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__global__ __launch_bounds__(256) void k_read(const uint4 *src, uint64_t n16, uint32_t *sink) {
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = per * blockIdx.x, hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0;
    uint64_t i = lo + threadIdx.x;
    for (; i + 3 * 256 < hi; i += 4 * 256) {
        const uint4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < hi; i += 256) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;  // almost never taken
}

}  // namespace

extern "C" int bench_read_launch(const void *src, uint64_t bytes, uint32_t *sink, int blocks, void *stream) {
    hipLaunchKernelGGL(k_read, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}
