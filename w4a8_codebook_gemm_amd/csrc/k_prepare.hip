// Kernel 1: per-call activation preparation -- 256-block Hadamard rotation fused with
// per-token symmetric int8 quantisation.
//
// Model cards: "Qwen3.8-27B-W4A8 (for ComfyUI)", section "Model Overview" (4-bit weights,
// int8 activations; Hadamard rotation in 256-blocks) and "Qwen3.8-27B-uncensored-w4a8-
// convrot-ComfyUI", section "Format" (rotation group 256; executed on int8 GEMM).  The
// activations take the same rotation as the weights' in_features so that the rotated
// product equals the original one (the orthonormal Sylvester transform is its own
// inverse).
//
// One workgroup of 16 waves per token row.  A wave owns whole 256-blocks: lane l holds
// elements 4l..4l+3 of a block in registers, so the transform's spans 1 and 2 are
// in-lane and spans 4..128 are lane-xor exchanges of distance 1..32.  Every butterfly is
// one fp32 add and one fp32 subtract in the fixed stage order 1, 2, 4, ..., 128, then the
// exact x 1/16: the int8 result is bit-reproducible.  Rows of up to 16 waves x 5 blocks
// (K <= 20480) stay in registers between the amax reduction and the quantisation;
// longer rows are rotated twice (identical arithmetic) instead of being stored.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kRegBlocks = 5;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_prepare(const void *__restrict__ x, int64_t K,
                                                      int8_t *__restrict__ xq,
                                                      float *__restrict__ sx) {
    __shared__ float red[kWaves];
    const int64_t m = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nblk = (int)(K / kRot);
    const int64_t row = m * K;
    const bool in_regs = nblk <= kWaves * kRegBlocks;

    float keep[kRegBlocks][4];
    float amax = 0.0f;
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kRegBlocks; i++) {
            const int b = wave + i * kWaves;
            if (b < nblk) {
                load4<BF16>(x, row + (int64_t)b * kRot + 4 * lane, keep[i]);
                fwht256_lane4(keep[i], lane);
#pragma unroll
                for (int q = 0; q < 4; q++) amax = fmaxf(amax, fabsf(keep[i][q]));
            }
        }
    } else {
        for (int b = wave; b < nblk; b += kWaves) {
            float v[4];
            load4<BF16>(x, row + (int64_t)b * kRot + 4 * lane, v);
            fwht256_lane4(v, lane);
#pragma unroll
            for (int q = 0; q < 4; q++) amax = fmaxf(amax, fabsf(v[q]));
        }
    }
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; w++) amax = fmaxf(amax, red[w]);

    const float s = amax / 127.0f;
    if (threadIdx.x == 0) sx[m] = s;
    uint32_t *out = reinterpret_cast<uint32_t *>(xq + row);
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kRegBlocks; i++) {
            const int b = wave + i * kWaves;
            if (b < nblk) out[(b * kRot) / 4 + lane] = (amax > 0.0f) ? quant4(keep[i], s) : 0u;
        }
    } else {
        for (int b = wave; b < nblk; b += kWaves) {
            float v[4];
            load4<BF16>(x, row + (int64_t)b * kRot + 4 * lane, v);
            fwht256_lane4(v, lane);
            out[(b * kRot) / 4 + lane] = (amax > 0.0f) ? quant4(v, s) : 0u;
        }
    }
}

}  // namespace

hipError_t launch_prepare(const void *x, int x_bf16, int64_t M, int64_t K, int8_t *x_q,
                          float *s_x, hipStream_t stream) {
    dim3 grid((unsigned)M), block(kThreads);
    if (x_bf16)
        hipLaunchKernelGGL(k_prepare<true>, grid, block, 0, stream, x, K, x_q, s_x);
    else
        hipLaunchKernelGGL(k_prepare<false>, grid, block, 0, stream, x, K, x_q, s_x);
    return hipGetLastError();
}

}  // namespace w4a8
