// Comparator: the W8A8 ("INT8 ConvRot") linear layer the W4A8 format is weighed against.
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", section "Why this exists": an
// INT8 ConvRot build of the same model takes about twice the weight bytes, and W4A8 runs on
// the same int8 GEMM path with a codebook dequantisation step added, so its only gain is
// the smaller weight stream.  The comparator keeps everything of the W4A8 layer except the
// weight format: the same 256-block Hadamard rotation and per-token int8 activations, and
// int8 weights w_q [N][K] with one fp32 scale per row (the rotated row's max |w| / 127).
//
//   y[m][r] = (fp32(sum_k x_q[m][k] * w_q[r][k]) * s_w[r]) * s_x[m]
//
// The integer sums are exact in int32 (|sum| <= 127^2 K < 2^31 for K <= 131072), so only
// the three fp32 roundings of the epilogue separate y from the exact value.
//
// Kernel W1 (decode, M <= 4): a persistent streaming GEMV.  Each workgroup owns an even
// share of the rows and stages all M activation rows in LDS; each wave walks a contiguous
// run of 1 KB row chunks (one 16-byte load per lane: eight whole 128-byte lines per load
// instruction), two batches of four chunks in flight, four v_dot4_i32_i8 per chunk and
// token.  A wave folds its lane sums with a butterfly when it leaves a row and adds them to
// the row's int32 accumulator in LDS (integer adds: the result does not depend on order).
//
// Kernel W2 (prefill): int8 MFMA GEMM, v_mfma_i32_32x32x32_i8, 256 tokens x 192 rows per
// 512-thread workgroup (4 x 2 waves of 64 x 96), one workgroup per CU, int32 accumulation
// over all of K, scales applied once in the epilogue.  The skeleton is the W4A8 prefill
// kernel's on requantised weights, so that the two compare like for like: 128-byte K
// stages double-buffered through LDS in 144-byte rows, global loads of whole 128-byte lines
// (eight lanes per row, eight rows per load) one stage ahead in a ring of two register
// stages, and a hand-scheduled stage in which the fragments of 32-k step t + 1 are read,
// and the next stage's rows stored, while step t's MFMAs run.  Tiles are numbered so that
// each XCD works through a contiguous run of them, token tiles fastest, which keeps a
// weight tile's reuse within one XCD's L2.
#include <type_traits>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

// ---------------------------------------------------------------- W1: decode GEMV
constexpr int kGvThreads = 1024, kGvWaves = kGvThreads / 64;
constexpr int kChunk = 1024;        // row bytes covered by one 16-byte load per lane
constexpr int kDepth = 4;           // chunks per batch of loads (two batches in flight)
constexpr int kGvMaxRows = 2048;    // rows per workgroup (int32 accumulators in LDS)

template <int MT>
__device__ __forceinline__ void fetch_batch(uint4 (&w)[kDepth], const int8_t *wrow, int64_t K,
                                            int &lrow, int &lc, int KC, int u, int u1, int kb_lane) {
#pragma unroll
    for (int d = 0; d < kDepth; d++) {
        const int kb = lc * kChunk + kb_lane;
        if (u + d < u1 && kb < K)
            w[d] = *reinterpret_cast<const uint4 *>(wrow + (int64_t)lrow * K + kb);
        else
            w[d] = make_uint4(0u, 0u, 0u, 0u);
        if (++lc == KC) {
            lc = 0;
            lrow++;
        }
    }
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

template <int MT>
__device__ __forceinline__ void consume_batch(const uint4 (&w)[kDepth], const int8_t *xs, int64_t K,
                                              int &crow, int &cc, int KC, int u, int u1, int kb_lane,
                                              int (&acc)[MT], bool &pending, int *accs, int lane) {
#pragma unroll
    for (int d = 0; d < kDepth; d++) {
        if (u + d >= u1) break;
        int kx = cc * kChunk + kb_lane;
        if (kx > K - 16) kx = (int)K - 16;   // lanes past the row end hold zero weights
#pragma unroll
        for (int m = 0; m < MT; m++) {
            const uint4 x = *reinterpret_cast<const uint4 *>(xs + (int64_t)m * K + kx);
            int s = acc[m];
            s = __builtin_amdgcn_sdot4((int)w[d].x, (int)x.x, s, false);
            s = __builtin_amdgcn_sdot4((int)w[d].y, (int)x.y, s, false);
            s = __builtin_amdgcn_sdot4((int)w[d].z, (int)x.z, s, false);
            s = __builtin_amdgcn_sdot4((int)w[d].w, (int)x.w, s, false);
            acc[m] = s;
        }
        pending = true;
        if (++cc == KC) {
#pragma unroll
            for (int m = 0; m < MT; m++) {
                const int v = wave_sum(acc[m]);
                if (lane == 0) atomicAdd(&accs[crow * MT + m], v);
                acc[m] = 0;
            }
            pending = false;
            cc = 0;
            crow++;
        }
    }
}

template <int MT>
__global__ __launch_bounds__(kGvThreads) void k_w8_gemv(W8Args a) {
    __shared__ __align__(16) int8_t xs[kW8GemvMaxX];
    __shared__ int accs[kGvMaxRows * MT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t K = a.K, N = a.N;
    const int64_t r0 = N * blockIdx.x / gridDim.x, r1 = N * (blockIdx.x + 1) / gridDim.x;
    const int R = (int)(r1 - r0);

    const int64_t nx = (int64_t)MT * K / 16;
    for (int64_t i = tid; i < nx; i += kGvThreads)
        reinterpret_cast<uint4 *>(xs)[i] = reinterpret_cast<const uint4 *>(a.x_q)[i];
    for (int i = tid; i < R * MT; i += kGvThreads) accs[i] = 0;
    __syncthreads();

    const int KC = (int)((K + kChunk - 1) / kChunk);
    const int U = R * KC;
    const int u0 = (int)((int64_t)U * wave / kGvWaves), u1 = (int)((int64_t)U * (wave + 1) / kGvWaves);
    const int kb_lane = lane * 16;
    const int8_t *wrow = a.w_q + r0 * K;

    int lrow = u0 / KC, lc = u0 - lrow * KC;   // next chunk to load
    int crow = lrow, cc = lc;                  // next chunk to consume
    int acc[MT];
#pragma unroll
    for (int m = 0; m < MT; m++) acc[m] = 0;
    bool pending = false;

    uint4 wa[kDepth], wb[kDepth];
    fetch_batch<MT>(wa, wrow, K, lrow, lc, KC, u0, u1, kb_lane);
    for (int u = u0; u < u1; u += 2 * kDepth) {
        fetch_batch<MT>(wb, wrow, K, lrow, lc, KC, u + kDepth, u1, kb_lane);
        consume_batch<MT>(wa, xs, K, crow, cc, KC, u, u1, kb_lane, acc, pending, accs, lane);
        fetch_batch<MT>(wa, wrow, K, lrow, lc, KC, u + 2 * kDepth, u1, kb_lane);
        consume_batch<MT>(wb, xs, K, crow, cc, KC, u + kDepth, u1, kb_lane, acc, pending, accs, lane);
    }
    if (pending) {   // the wave's run ended inside a row
#pragma unroll
        for (int m = 0; m < MT; m++) {
            const int v = wave_sum(acc[m]);
            if (lane == 0) atomicAdd(&accs[crow * MT + m], v);
        }
    }
    __syncthreads();

    for (int i = tid; i < R * MT; i += kGvThreads) {
        const int m = i / R, row = i - m * R;
        const int64_t r = r0 + row;
        const float v = ((float)accs[row * MT + m] * a.s_w[r]) * a.s_x[m];
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[m * N + r] = f32_to_bf16_rne(v);
        else
            static_cast<float *>(a.y)[m * N + r] = v;
    }
}

// ---------------------------------------------------------------- W2: prefill GEMM
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));

constexpr int GM = 256, GN = 192, GK = 128;  // tile: tokens x weight rows x K bytes per stage
constexpr int kGmThreads = 512;
constexpr int GJB = GN / 64;                // 32-row weight blocks per wave
// 144-byte LDS rows: the 16 rows one 16-lane phase of a 16-byte fragment read touches start
// on distinct bank quads of the 64 banks
constexpr int kPitch = GK + 16;
constexpr int kXSt = GM * kPitch, kWSt = GN * kPitch;
constexpr int XJ = GM / 64, WJ = GN / 64;   // staged rows per thread: 4 activation, 3 weight

struct GStage {
    int4v x[XJ];   // 16 activation bytes of rows sr + 64 j
    int4v w[WJ];   // 16 weight bytes of rows sr + 64 j
};

struct GFrag {
    int4v A[2], B[GJB];
};

template <int J>
using GIC = std::integral_constant<int, J>;

// two waves per SIMD: the accumulators, two fragment sets and the register ring
__global__ __launch_bounds__(kGmThreads, 1) void k_w8_gemm(W8Args a, int tiles_m, int tiles) {
    __shared__ __align__(16) int8_t xs[2 * kXSt];
    __shared__ __align__(16) int8_t ws[2 * kWSt];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;

    // consecutive workgroups go to consecutive XCDs: give XCD x the contiguous tile run
    // [x*q + min(x, rem), ...) so that neighbouring tiles share an L2
    const int b = blockIdx.x, q = tiles / 8, rem = tiles % 8, xcd = b % 8, slot = b / 8;
    const int t = xcd * q + min(xcd, rem) + slot;
    const int64_t m0 = (int64_t)(t % tiles_m) * GM, n0 = (int64_t)(t / tiles_m) * GN;

    // staging: rows sr + 64 j, 16-byte chunk sc of the stage.  Rows past M or N re-read the
    // last valid row: they feed only outputs that are never stored.
    const int sr = tid >> 3, sc = tid & 7;
    const int8_t *xp[XJ];
    const int8_t *wp[WJ];
#pragma unroll
    for (int j = 0; j < XJ; j++) xp[j] = a.x_q + min<int64_t>(m0 + sr + 64 * j, M - 1) * K + 16 * sc;
#pragma unroll
    for (int j = 0; j < WJ; j++) wp[j] = a.w_q + min<int64_t>(n0 + sr + 64 * j, N - 1) * K + 16 * sc;
    const int nk = (int)(K / GK);  // even: K is a multiple of 256

    // every stage's loads are issued unconditionally (stages past the end re-read the last
    // one) so that the in-order load counter lets a store wait for its own stage only
    auto gload = [&](int kt, GStage &st) {
        const int64_t k = (int64_t)(kt < nk ? kt : nk - 1) * GK;
#pragma unroll
        for (int j = 0; j < XJ; j++) st.x[j] = *reinterpret_cast<const int4v *>(xp[j] + k);
#pragma unroll
        for (int j = 0; j < WJ; j++) st.w[j] = *reinterpret_cast<const int4v *>(wp[j] + k);
    };
    auto xstore = [&](int buf, const GStage &st) {
#pragma unroll
        for (int j = 0; j < XJ; j++)
            *reinterpret_cast<int4v *>(&xs[buf * kXSt + (sr + 64 * j) * kPitch + 16 * sc]) = st.x[j];
    };
    auto wstore = [&](int buf, int j, const GStage &st) {
        *reinterpret_cast<int4v *>(&ws[buf * kWSt + (sr + 64 * j) * kPitch + 16 * sc]) = st.w[j];
    };

    int16v acc[2][GJB];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < GJB; j++) acc[i][j] = int16v{};

    GStage R0, R1;
    gload(0, R0);
    gload(1, R1);
    xstore(0, R0);
#pragma unroll
    for (int j = 0; j < WJ; j++) wstore(0, j, R0);
    __syncthreads();

    const int half = lane >> 5, l32 = lane & 31;
    const int8_t *const xrd = &xs[(wm * 64 + l32) * kPitch + 16 * half];
    const int8_t *const wrd = &ws[(wn * (GN / 2) + l32) * kPitch + 16 * half];
    // A and B lanes carry the same 16 k of a 32-wide step, so the product is the full sum
    // over the step whatever order the unit takes them in
    auto frag = [&](int buf, int s, GFrag &f) {
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
            f.A[ib] = *reinterpret_cast<const int4v *>(xrd + buf * kXSt + ib * 32 * kPitch + s * 32);
#pragma unroll
        for (int jb = 0; jb < GJB; jb++)
            f.B[jb] = *reinterpret_cast<const int4v *>(wrd + buf * kWSt + jb * 32 * kPitch + s * 32);
    };
    auto mma = [&](const GFrag &f) {
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
#pragma unroll
            for (int jb = 0; jb < GJB; jb++)
                acc[ib][jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.A[ib], f.B[jb], acc[ib][jb], 0, 0, 0);
    };
    // One stage: the MFMAs of buffer cur (four 32-k steps) while stage data nx is stored
    // into buffer cur ^ 1.  The scheduling barriers keep the fragments of step t + 1 (and a
    // share of the stores) ahead of step t's MFMAs.
    auto stage = [&](auto curc, const GStage &nx) {
        constexpr int cur = decltype(curc)::value, oth = cur ^ 1;
        GFrag F0, F1;
        frag(cur, 0, F0);
        __builtin_amdgcn_sched_barrier(0);
        xstore(oth, nx);
        frag(cur, 1, F1);
        __builtin_amdgcn_sched_barrier(0);
        mma(F0);
        __builtin_amdgcn_sched_barrier(0);
        wstore(oth, 0, nx);
        frag(cur, 2, F0);
        __builtin_amdgcn_sched_barrier(0);
        mma(F1);
        __builtin_amdgcn_sched_barrier(0);
        wstore(oth, 1, nx);
        frag(cur, 3, F1);
        __builtin_amdgcn_sched_barrier(0);
        mma(F0);
        __builtin_amdgcn_sched_barrier(0);
        wstore(oth, 2, nx);
        __builtin_amdgcn_sched_barrier(0);
        mma(F1);
    };
    // stage s is in LDS buffer s % 2 and stage s + 1 in ring slot (s + 1) % 2; the slot of
    // stage s (already stored) is reloaded with stage s + 2 first
    for (int s = 0; s < nk; s += 2) {
        gload(s + 2, R0);
        stage(GIC<0>{}, R1);
        __syncthreads();
        gload(s + 3, R1);
        stage(GIC<1>{}, R0);
        __syncthreads();
    }

    // lane holds weight row j = l32 of each 32 x 32 block and tokens 8(v/4) + 4 half + v%4
#pragma unroll
    for (int jb = 0; jb < GJB; jb++) {
        const int64_t r = n0 + wn * (GN / 2) + jb * 32 + l32;
        if (r >= N) continue;
        const float sw = a.s_w[r];
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t m = m0 + wm * 64 + ib * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                if (m < M) {
                    const float val = ((float)acc[ib][jb][v] * sw) * a.s_x[m];
                    if (a.y_bf16)
                        static_cast<uint16_t *>(a.y)[m * N + r] = f32_to_bf16_rne(val);
                    else
                        static_cast<float *>(a.y)[m * N + r] = val;
                }
            }
    }
}

}  // namespace

bool w8_gemv_supported(int64_t M, int64_t K) { return M >= 1 && M <= 4 && M * K <= kW8GemvMaxX; }

hipError_t launch_w8_gemv(const W8Args &a, int num_cu, hipStream_t stream) {
    int64_t grid = num_cu;
    const int64_t need = (a.N + kGvMaxRows - 1) / kGvMaxRows;
    if (grid < need) grid = need;
    switch (a.M) {
        case 1: hipLaunchKernelGGL(k_w8_gemv<1>, dim3((unsigned)grid), dim3(kGvThreads), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(k_w8_gemv<2>, dim3((unsigned)grid), dim3(kGvThreads), 0, stream, a); break;
        case 3: hipLaunchKernelGGL(k_w8_gemv<3>, dim3((unsigned)grid), dim3(kGvThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL(k_w8_gemv<4>, dim3((unsigned)grid), dim3(kGvThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_w8_gemm(const W8Args &a, hipStream_t stream) {
    const int64_t tm = (a.M + GM - 1) / GM, tn = (a.N + GN - 1) / GN;
    hipLaunchKernelGGL(k_w8_gemm, dim3((unsigned)(tm * tn)), dim3(kGmThreads), 0, stream, a, (int)tm,
                       (int)(tm * tn));
    return hipGetLastError();
}

}  // namespace w4a8
