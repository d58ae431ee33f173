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
// Each 256-block belongs to one 16-lane DPP row (16 consecutive values per lane, see
// fwht256_row16): the rotation needs no LDS, and a lane's 16 results are 16 consecutive int8
// outputs (one 16-byte store).  The workgroup is sized to the row (16 lanes per block, at most
// 1024 threads).
//  * Rows of up to two blocks per lane group (K <= 32768): a workgroup works through tokens
//    blockIdx.x, blockIdx.x + gridDim.x, ... with a grid of about as many workgroups as the
//    CUs hold at once.  The next token's loads are issued before the current token is
//    rotated, reduced and quantised, so every workgroup keeps a token's loads in flight
//    behind its work (one workgroup per token left a CU with one 68 KiB token in flight at
//    K = 17408, and the launch ran as eight latency-bound rounds).  The workgroup maximum
//    goes through an LDS slot per token parity: one barrier per token.
//  * Longer rows: one workgroup per token, rotated twice (identical arithmetic) instead of
//    being stored.
#include <atomic>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kRegRounds = 2;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOutside = 0x80000000u;  // buffer offset past any row: reads zero, stores dropped
constexpr int kRsrcWord3 = 0x00020000;      // buffer resource: raw 32-bit elements

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

// Tokens m = blockIdx.x + i * gridDim.x of rows with R <= 2 blocks per lane group: the
// arithmetic of k_prepare.  Every token row is addressed through a buffer resource of its own
// (a token past the last gets an empty one), so an absent block or token reads as zeros and
// its stores are dropped, with no branch around any load or store: the wait before a token's
// rotation then counts only that token's loads, and the next token's stay in flight.  (With
// the loads under a branch, the wait took the count of the path without them and drained the
// next token's loads as well.)
template <bool BF16, int R>
__global__ __launch_bounds__(kMaxThreads) void k_prepare_tokens(const void *__restrict__ x, int64_t M, int64_t K,
                                                                int8_t *__restrict__ xq,
                                                                float *__restrict__ sx) {
    __shared__ float red[2][kMaxThreads / 64];
    constexpr int kEs = BF16 ? 2 : 4;  // bytes per input element
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const int groups = blockDim.x >> 4;
    const int g = tid >> 4, t = tid & 15;
    const int h = fwht_row16_nibble(t);
    const int nblk = (int)(K / kRot);

    // per round: byte offsets of this lane's 16 values in an input row and in an output row
    uint32_t xo[R], qo[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int b = g + r * groups;
        const uint32_t e = (uint32_t)(b * kRot + 16 * h);
        xo[r] = b < nblk ? e * kEs : kOutside;
        qo[r] = b < nblk ? e : kOutside;
    }
    auto row = [&](const void *base, int64_t m, int64_t bytes) {
        const bool in = m < M;
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(static_cast<const char *>(base) + (in ? m : 0) * bytes), (short)0, in ? (int)bytes : 0, kRsrcWord3);
    };
    // plain (temporal) loads: a lane's four 16-byte loads cover 64 consecutive bytes, and one
    // load instruction of a row touches every other 32 bytes of its lines, so a line serves
    // several loads (non-temporal loads ran 30% slower)
    auto load = [&](int64_t m, float (&v)[R][16]) {
        const __amdgpu_buffer_rsrc_t rs = row(x, m, K * kEs);
#pragma unroll
        for (int r = 0; r < R; r++) {
            if constexpr (BF16) {
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, xo[r], 0, 0);
                const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, xo[r] + 16u, 0, 0);
                const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    v[r][2 * i] = __uint_as_float(w[i] << 16);
                    v[r][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const u32x4 f = __builtin_amdgcn_raw_buffer_load_b128(rs, xo[r] + 16u * i, 0, 0);
                    v[r][4 * i] = __uint_as_float(f.x); v[r][4 * i + 1] = __uint_as_float(f.y);
                    v[r][4 * i + 2] = __uint_as_float(f.z); v[r][4 * i + 3] = __uint_as_float(f.w);
                }
            }
        }
    };
    auto finish = [&](int64_t m, float (&v)[R][16], int par) {
        // an absent block is all zeros: its rotation is zero and leaves the maximum alone
        float amax = 0.0f;
#pragma unroll
        for (int r = 0; r < R; r++) {
            fwht256_row16(v[r], t);
#pragma unroll
            for (int q = 0; q < 16; q++) amax = fmaxf(amax, fabsf(v[r][q]));
        }
#pragma unroll
        for (int sh = 32; sh > 0; sh >>= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
        if (lane == 0) red[par][wave] = amax;
        __syncthreads();
        amax = red[par][0];
        for (int w = 1; w < nwaves; w++) amax = fmaxf(amax, red[par][w]);
        const float s = amax / 127.0f;
        const float rs = s >= kQuantFastMin ? 1.0f / s : 0.0f;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), row(sx, m, 4), tid == 0 ? 0u : kOutside, 0, 0);
        const __amdgpu_buffer_rsrc_t rq = row(xq, m, K);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const uint4 q = (amax > 0.0f) ? quant16_auto(v[r], s, rs) : make_uint4(0, 0, 0, 0);
            u32x4 o;
            o.x = q.x; o.y = q.y; o.z = q.z; o.w = q.w;
            __builtin_amdgcn_raw_buffer_store_b128(o, rq, qo[r], 0, 0);
        }
    };

    // two register sets, alternating: the next token's loads are in flight while the current
    // one is finished (the LDS slot alternates with them: a workgroup's threads read red[par]
    // before the next token's barrier and write it again only one token later)
    float A[R][16], B[R][16];
    const int64_t step = gridDim.x;
    int64_t m = blockIdx.x;  // < M: the grid is at most M
    load(m, A);
    for (;;) {
        const int64_t m1 = m + step;
        load(m1, B);
        finish(m, A, 0);
        if (m1 >= M) break;
        load(m1 + step, A);
        finish(m1, B, 1);
        m = m1 + step;
        if (m >= M) break;
    }
}

template <bool BF16, int R>
hipError_t launch_tokens(const void *x, int64_t M, int64_t K, int8_t *x_q, float *s_x, int num_cu,
                         unsigned threads, hipStream_t stream) {
    // about as many workgroups as the CUs hold at once, each working through its share of the
    // tokens (workgroups per CU from the kernel's registers, looked up once per size)
    static std::atomic<int> per_cu[kMaxThreads / 64 + 1];
    int pc = per_cu[threads / 64].load(std::memory_order_relaxed);
    if (pc == 0) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, k_prepare_tokens<BF16, R>, (int)threads, 0);
        if (e != hipSuccess) return e;
        if (pc < 1) pc = 1;
        per_cu[threads / 64].store(pc, std::memory_order_relaxed);
    }
    int64_t grid = (int64_t)num_cu * pc;
    if (grid > M) grid = M;
    hipLaunchKernelGGL((k_prepare_tokens<BF16, R>), dim3((unsigned)grid), dim3(threads), 0, stream, x, M, K, x_q, s_x);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(const void *x, int x_bf16, int64_t M, int64_t K, int8_t *x_q,
                          float *s_x, int num_cu, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const int64_t nblk = K / kRot;
    const int64_t rounds = (nblk * 16 + kMaxThreads - 1) / kMaxThreads;  // 256-blocks per lane group
    if (rounds <= kRegRounds) {
        // 16 lanes per block and round, whole waves
        const unsigned threads = (unsigned)(((nblk + rounds - 1) / rounds * 16 + 63) / 64 * 64);
        if (rounds == 1)
            return x_bf16 ? launch_tokens<true, 1>(x, M, K, x_q, s_x, num_cu, threads, stream)
                          : launch_tokens<false, 1>(x, M, K, x_q, s_x, num_cu, threads, stream);
        return x_bf16 ? launch_tokens<true, 2>(x, M, K, x_q, s_x, num_cu, threads, stream)
                      : launch_tokens<false, 2>(x, M, K, x_q, s_x, num_cu, threads, stream);
    }
    dim3 grid((unsigned)M), block(kMaxThreads);
    if (x_bf16)
        hipLaunchKernelGGL(k_prepare<true>, grid, block, 0, stream, x, K, x_q, s_x);
    else
        hipLaunchKernelGGL(k_prepare<false>, grid, block, 0, stream, x, K, x_q, s_x);
    return hipGetLastError();
}

}  // namespace w4a8
