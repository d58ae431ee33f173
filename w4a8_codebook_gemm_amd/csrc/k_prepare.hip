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
// One workgroup per token row.  Each 256-block belongs to one 16-lane DPP row (16
// consecutive values per lane, see fwht256_row16): the rotation needs no LDS, and a lane's
// 16 results are 16 consecutive int8 outputs (one 16-byte store).  The workgroup is sized to
// the row (16 lanes per block, at most 1024 threads); every block's loads are issued before
// the first rotation so their latencies overlap.  Rows of up to two blocks per lane group
// (K <= 32768) stay in registers between the amax reduction and the quantisation; longer
// rows are rotated twice (identical arithmetic) instead of being stored.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kRegRounds = 2;

template <bool BF16>
__global__ __launch_bounds__(kMaxThreads) void k_prepare(const void *__restrict__ x, int64_t K,
                                                         int8_t *__restrict__ xq,
                                                         float *__restrict__ sx) {
    __shared__ float red[kMaxThreads / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const int groups = blockDim.x >> 4;           // 16-lane rows, one 256-block each per round
    const int g = tid >> 4, t = tid & 15;
    const int h = fwht_row16_nibble(t);
    const int nblk = (int)(K / kRot);
    const int rounds = (nblk + groups - 1) / groups;
    const int64_t row = m * K;
    const bool in_regs = rounds <= kRegRounds;

    float keep[kRegRounds][16];
    float amax = 0.0f;
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < kRegRounds; r++) {
            const int b = g + r * groups;
            if (b < nblk) {
                load16<BF16>(x, row + (int64_t)b * kRot + 16 * h, keep[r]);
            } else {
#pragma unroll
                for (int q = 0; q < 16; q++) keep[r][q] = 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < kRegRounds; r++) {
            if (g + r * groups < nblk) {  // whole 16-lane rows: absent blocks skip the rotation
                fwht256_row16(keep[r], t);
#pragma unroll
                for (int q = 0; q < 16; q++) amax = fmaxf(amax, fabsf(keep[r][q]));
            }
        }
    } else {
        for (int r = 0; r < rounds; r++) {
            const int b = g + r * groups;
            float v[16];
            if (b < nblk) {
                load16<BF16>(x, row + (int64_t)b * kRot + 16 * h, v);
            } else {
#pragma unroll
                for (int q = 0; q < 16; q++) v[q] = 0.0f;
            }
            fwht256_row16(v, t);
#pragma unroll
            for (int q = 0; q < 16; q++) amax = fmaxf(amax, fabsf(v[q]));
        }
    }
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < nwaves; w++) amax = fmaxf(amax, red[w]);

    const float s = amax / 127.0f;
    const float rs = s >= kQuantFastMin ? 1.0f / s : 0.0f;
    if (tid == 0) sx[m] = s;
    uint4 *out = reinterpret_cast<uint4 *>(xq + row);
    const uint4 zero = make_uint4(0, 0, 0, 0);
    if (in_regs) {
#pragma unroll
        for (int r = 0; r < kRegRounds; r++) {
            const int b = g + r * groups;
            if (b < nblk) out[(b * kRot + 16 * h) / 16] = (amax > 0.0f) ? quant16_auto(keep[r], s, rs) : zero;
        }
    } else {
        for (int r = 0; r < rounds; r++) {
            const int b = g + r * groups;
            float v[16];
            if (b < nblk) {
                load16<BF16>(x, row + (int64_t)b * kRot + 16 * h, v);
            } else {
#pragma unroll
                for (int q = 0; q < 16; q++) v[q] = 0.0f;
            }
            fwht256_row16(v, t);
            if (b < nblk) out[(b * kRot + 16 * h) / 16] = (amax > 0.0f) ? quant16_auto(v, s, rs) : zero;
        }
    }
}

}  // namespace

hipError_t launch_prepare(const void *x, int x_bf16, int64_t M, int64_t K, int8_t *x_q,
                          float *s_x, hipStream_t stream) {
    // 16 lanes per 256-block, whole waves, at most kMaxThreads
    const int64_t want = ((K / kRot) * 16 + 63) / 64 * 64;
    const unsigned threads = (unsigned)(want < kMaxThreads ? want : kMaxThreads);
    dim3 grid((unsigned)M), block(threads);
    if (x_bf16)
        hipLaunchKernelGGL(k_prepare<true>, grid, block, 0, stream, x, K, x_q, s_x);
    else
        hipLaunchKernelGGL(k_prepare<false>, grid, block, 0, stream, x, K, x_q, s_x);
    return hipGetLastError();
}

}  // namespace w4a8
