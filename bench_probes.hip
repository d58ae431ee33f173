// Measurement helpers for bench.py (not part of the library): the ceilings the library's
// kernels are set beside.
//
//  * bench_read_launch: the achievable HBM read rate for a byte count.  One workgroup per
//    compute unit (or a few) reads a contiguous share of the buffer with non-temporal
//    16-byte buffer loads, DEPTH loads in flight per thread, and folds what it read into
//    one word that it stores only in a case that never happens, so the loads cannot be
//    dropped.  The benchmark sweeps workgroup width, depth and workgroups per unit and keeps
//    the fastest.
//  * bench_stream_launch: the achievable rate of a streaming read + write in the activation
//    preparation's proportion, four bytes read per byte written (fp32 in, int8 out).  Each
//    workgroup converts a contiguous share: a 16-byte load per thread and step (DEPTH steps
//    in flight), a 4-byte store of its low bytes.
//
// Both take device pointers, launch on the given stream and return the HIP error code of
// the launch.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int THREADS, int DEPTH>
__global__ __launch_bounds__(THREADS) void k_read(const uint8_t *src, uint64_t n16, uint32_t *sink) {
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;      // 16-byte chunks per workgroup
    const uint64_t lo = per * blockIdx.x, hi = lo + per < n16 ? lo + per : n16;
    const uint64_t cnt = hi > lo ? hi - lo : 0;
    // the workgroup's share as a buffer resource: chunks past its end read as zero
    const uint64_t bytes = cnt * 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(src + lo * 16), (short)0, (int)(bytes < 0x7FFFFFFFull ? bytes : 0x7FFFFFFFull), 0x00020000);
    uint32_t acc = 0;
    for (uint64_t i = threadIdx.x; i < cnt; i += (uint64_t)DEPTH * THREADS) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; d++)
            v[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((i + (uint64_t)d * THREADS) * 16), 0, 2);
#pragma unroll
        for (int d = 0; d < DEPTH; d++) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x * THREADS + threadIdx.x] = acc;  // almost never taken
}

template <int THREADS, int DEPTH>
int launch_read(const void *src, uint64_t bytes, uint32_t *sink, int blocks, hipStream_t s) {
    hipLaunchKernelGGL((k_read<THREADS, DEPTH>), dim3((unsigned)blocks), dim3(THREADS), 0, s,
                       static_cast<const uint8_t *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}

template <int THREADS, int DEPTH>
__global__ __launch_bounds__(THREADS) void k_stream(const uint8_t *src, uint64_t n16, uint8_t *dst) {
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = per * blockIdx.x, hi = lo + per < n16 ? lo + per : n16;
    const uint64_t cnt = hi > lo ? hi - lo : 0;
    // the share as buffer resources: loads past its end read zero, stores past it are dropped
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)(src + lo * 16), (short)0,
                                                                        (int)(cnt * 16), 0x00020000);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void *)(dst + lo * 4), (short)0,
                                                                        (int)(cnt * 4), 0x00020000);
    for (uint64_t i = threadIdx.x; i < cnt; i += (uint64_t)DEPTH * THREADS) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; d++)
            v[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((i + (uint64_t)d * THREADS) * 16), 0, 0);
#pragma unroll
        for (int d = 0; d < DEPTH; d++) {
            const uint32_t w = __builtin_amdgcn_perm(__builtin_amdgcn_perm(v[d].w, v[d].z, 0x0c0c0400u),
                                                     __builtin_amdgcn_perm(v[d].y, v[d].x, 0x0c0c0400u), 0x05040100u);
            __builtin_amdgcn_raw_buffer_store_b32(w, rd, (uint32_t)((i + (uint64_t)d * THREADS) * 4), 0, 0);
        }
    }
}

template <int THREADS, int DEPTH>
int launch_stream(const void *src, uint64_t bytes, void *dst, int blocks, hipStream_t s) {
    hipLaunchKernelGGL((k_stream<THREADS, DEPTH>), dim3((unsigned)blocks), dim3(THREADS), 0, s,
                       static_cast<const uint8_t *>(src), bytes / 16, static_cast<uint8_t *>(dst));
    return (int)hipGetLastError();
}

}  // namespace

// threads in {256, 512, 1024}, depth in {1, 2, 4, 8}; bytes a multiple of 16, and a
// workgroup's share below 2 GiB (the buffer resource's range).  Returns -1 for another
// width or depth.
extern "C" int bench_read_launch(const void *src, uint64_t bytes, uint32_t *sink, int blocks, int threads,
                                 int depth, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
#define W4A8_READ_CASE(T, D) if (threads == T && depth == D) return launch_read<T, D>(src, bytes, sink, blocks, s);
    W4A8_READ_CASE(256, 1) W4A8_READ_CASE(256, 2) W4A8_READ_CASE(256, 4) W4A8_READ_CASE(256, 8)
    W4A8_READ_CASE(512, 1) W4A8_READ_CASE(512, 2) W4A8_READ_CASE(512, 4) W4A8_READ_CASE(512, 8)
    W4A8_READ_CASE(1024, 1) W4A8_READ_CASE(1024, 2) W4A8_READ_CASE(1024, 4) W4A8_READ_CASE(1024, 8)
#undef W4A8_READ_CASE
    return -1;
}

// src holds `bytes` (a multiple of 16) and dst bytes / 4; a workgroup's share below 2 GiB.
// threads in {256, 512, 1024}, depth in {1, 2, 4}; -1 for another width or depth.
extern "C" int bench_stream_launch(const void *src, uint64_t bytes, void *dst, int blocks, int threads, int depth,
                                   void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
#define W4A8_STREAM_CASE(T, D) if (threads == T && depth == D) return launch_stream<T, D>(src, bytes, dst, blocks, s);
    W4A8_STREAM_CASE(256, 1) W4A8_STREAM_CASE(256, 2) W4A8_STREAM_CASE(256, 4)
    W4A8_STREAM_CASE(512, 1) W4A8_STREAM_CASE(512, 2) W4A8_STREAM_CASE(512, 4)
    W4A8_STREAM_CASE(1024, 1) W4A8_STREAM_CASE(1024, 2) W4A8_STREAM_CASE(1024, 4)
#undef W4A8_STREAM_CASE
    return -1;
}
