// Kernel 3a': prefill GEMM on int8 MFMA with the per-16 group scales folded into the exact
// int32 partial sums, step by step as the pages describe the int8 path (the explicit
// algorithm W4A8_ALGO_MFMA_I8_FOLD; the int8-codebook route W4A8_ALGO_MFMA_I8 computes the
// same products with the group scale folded exactly into an fp16 weight instead).
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", sections "Why this exists"
// and "Format": the W4A8 layer runs on the same int8 GEMM path as INT8 and adds a
// codebook dequantisation step; int4 indices, a per-tensor 16-level codebook, an e4m3
// scale per 16 values and an fp32 scale per output row.
//
// The fp32 codebook is carried on the int8 path as s_cb = max|cb| / 127 and
// cb_i8 = rint(cb / s_cb).  One v_mfma_i32_32x32x16_i8 covers exactly one group of 16
// along K, so its int32 outputs are the exact partials P[m, r, g] = sum x_q * cb_i8[idx];
// each is converted to fp32 and folded with its group scale: acc += dec(s_rel[r, g]) * P.
// The weight rows are the MFMA's N side, so all 16 accumulators of a lane belong to one
// weight row and share one group scale.  y = acc * s_cb * s_channel[r] * s_x[m].
//
// The fold (one conversion and one fma per partial) is the kernel's bound: it costs more
// vector-ALU time than the MFMA takes, so everything else is kept off the vector ALU.
// Tile: 256 tokens x 192 weight rows per 512-thread workgroup, one workgroup per CU.
// Waves 4 (tokens) x 2 (rows), each 64 x 96 = 2 x 3 MFMA blocks.  K advances in stages of
// 64 (four groups), double-buffered through LDS, with the global loads four stages ahead in
// a ring of register stages.  Per stage the workgroup
//  * copies the int8 activations into [token][64 + 8 pad] rows;
//  * decodes the packed indices once into int8 weights (byte-permute lookups in a
//    16-byte cb_i8 table held in registers) in [row][64 + 8 pad] rows;
//  * decodes the group scales once into fp32 [group][row].
// The 72-byte rows put the 32 rows one 32-lane phase of an 8-byte fragment read touches on
// distinct 8-byte bank pairs of the 64 banks.  Tiles are numbered so that each XCD works
// through a contiguous run, token tiles fastest.
#include <type_traits>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int int16v __attribute__((ext_vector_type(16)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 192, BK = 64;
constexpr int kThreads = 512;
constexpr int JB = BN / 64;                    // 32-row weight blocks per wave
constexpr int kPitch = BK + 8;                 // bytes per LDS row
constexpr int kXStage = BM * kPitch, kBStage = BN * kPitch, kSStage = (BK / kGroup) * BN;

struct Stage {
    uint4 x0, x1;   // 32 activation bytes of token xr
    uint4 p;        // 32 packed indices of weight row pr (two groups)
    uint32_t s;     // the four e4m3 group scales of weight row sr (threads < BN)
};

template <int J>
using IC = std::integral_constant<int, J>;

__global__ __launch_bounds__(kThreads) void k_gemm_i8_fold(LinearArgs a, int tiles_m, int tiles) {
    __shared__ __align__(16) int8_t xs[2][kXStage];
    __shared__ __align__(16) int8_t bs[2][kBStage];
    __shared__ __align__(16) float ss[2][kSStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;

    // consecutive workgroups go to consecutive XCDs: XCD x takes the contiguous tile run
    // starting at x*q + min(x, rem)
    const int b = blockIdx.x, q = tiles / 8, rem = tiles % 8, xcd = b % 8, slot = b / 8;
    const int t = xcd * q + min(xcd, rem) + slot;
    const int64_t m0 = (int64_t)(t % tiles_m) * BM, n0 = (int64_t)(t / tiles_m) * BN;

    // int8 form of the codebook (same fp32 arithmetic at every thread)
    float cmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kLevels; j++) cmax = fmaxf(cmax, fabsf(a.cb[j]));
    const float s_cb = cmax / 127.0f;
    CbI8 cbt;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        uint32_t v = 0;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
            const int qv = (s_cb > 0.0f) ? (int)rintf(a.cb[4 * w + bb] / s_cb) : 0;
            v |= ((uint32_t)qv & 0xFFu) << (8 * bb);
        }
        cbt.t[w] = v;
    }

    // ---- staging roles: token xr, bytes [32 xh, 32 xh + 32) of a stage; weight row pr,
    // weights [32 ph, 32 ph + 32) (two groups); group scales of row sr.  Rows past M or N
    // re-read the last valid row: they feed only outputs that are never stored.  Threads
    // past 2 BN (packed) or BN (scales) load like the last row's but store nothing.
    const int xr = tid >> 1, xh = tid & 1;
    const int pr0 = tid >> 1, ph = tid & 1;
    const bool pdec = pr0 < BN;                    // wave-uniform: 2 BN is a multiple of 64
    const int pr = pdec ? pr0 : BN - 1;
    const bool sdec = tid < BN;                    // wave-uniform: BN is a multiple of 64
    const int sr = sdec ? tid : BN - 1;
    const int8_t *xp = a.x_q + min<int64_t>(m0 + xr, M - 1) * K + 32 * xh;
    const int8_t *pp = a.packed + min<int64_t>(n0 + pr, N - 1) * (K / 2) + 16 * ph;
    // a row's group scales start 16-byte aligned (K / 16 is a multiple of 16); one dword
    // holds the stage's four
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(a.s_rel + min<int64_t>(n0 + sr, N - 1) * (K / kGroup));
    const int nk = (int)(K / BK);

    // every stage's loads are issued unconditionally (stages past the end re-read the last
    // one) so that the in-order load counter lets a decode wait for its own stage only
    auto gload = [&](int kt, Stage &st) {
        const int k = kt < nk ? kt : nk - 1;
        st.x0 = *reinterpret_cast<const uint4 *>(xp + (int64_t)k * BK);
        st.x1 = *reinterpret_cast<const uint4 *>(xp + (int64_t)k * BK + 16);
        st.p = *reinterpret_cast<const uint4 *>(pp + (int64_t)k * (BK / 2));
        st.s = sp[k];
    };
    int8_t *const xdst = &xs[0][xr * kPitch + 32 * xh];
    int8_t *const bdst = &bs[0][pr * kPitch + 32 * ph];
    auto lstore = [&](auto bufc, const Stage &st) {
        constexpr int buf = decltype(bufc)::value;
        // 72-byte rows: 8-byte stores
        uint2 *dx = reinterpret_cast<uint2 *>(xdst + buf * kXStage);
        dx[0] = make_uint2(st.x0.x, st.x0.y);
        dx[1] = make_uint2(st.x0.z, st.x0.w);
        dx[2] = make_uint2(st.x1.x, st.x1.y);
        dx[3] = make_uint2(st.x1.z, st.x1.w);
        if (pdec) {
            uint2 *db = reinterpret_cast<uint2 *>(bdst + buf * kBStage);
            db[0] = decode8(cbt, st.p.x);
            db[1] = decode8(cbt, st.p.y);
            db[2] = decode8(cbt, st.p.z);
            db[3] = decode8(cbt, st.p.w);
        }
        if (sdec) {
            // gfx950's v_cvt_f32_fp8 decodes OCP E4M3FN exactly
            float *dsc = &ss[buf][sr];
            dsc[0 * BN] = __builtin_amdgcn_cvt_f32_fp8((int)st.s, 0);
            dsc[1 * BN] = __builtin_amdgcn_cvt_f32_fp8((int)st.s, 1);
            dsc[2 * BN] = __builtin_amdgcn_cvt_f32_fp8((int)st.s, 2);
            dsc[3 * BN] = __builtin_amdgcn_cvt_f32_fp8((int)st.s, 3);
        }
    };

    float16_t acc[2][JB];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < JB; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    Stage R0, R1, R2, R3;
    gload(0, R0);
    gload(1, R1);
    gload(2, R2);
    gload(3, R3);
    lstore(IC<0>{}, R0);
    __syncthreads();

    const int half = lane >> 5, l32 = lane & 31;
    const int8_t *const xrd = &xs[0][(wm * 64 + l32) * kPitch + 8 * half];
    const int8_t *const brd = &bs[0][(wn * (BN / 2) + l32) * kPitch + 8 * half];
    const float *const srd = &ss[0][wn * (BN / 2) + l32];

    auto mfmas = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        // rolled on purpose: each group's partials are folded before the next group's
        // MFMAs issue, so only one group's partials are live at a time
#pragma unroll 1
        for (int g = 0; g < BK / kGroup; g++) {
            long A[2], B[JB];
            float s[JB];
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
                A[ib] = *reinterpret_cast<const long *>(xrd + buf * kXStage + ib * 32 * kPitch + g * kGroup);
#pragma unroll
            for (int jb = 0; jb < JB; jb++) {
                B[jb] = *reinterpret_cast<const long *>(brd + buf * kBStage + jb * 32 * kPitch + g * kGroup);
                s[jb] = srd[buf * kSStage + g * BN + jb * 32];
            }
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
#pragma unroll
                for (int jb = 0; jb < JB; jb++) {
                    const int16v zero = {};
                    const int16v P = __builtin_amdgcn_mfma_i32_32x32x16_i8(A[ib], B[jb], zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 16; v++) acc[ib][jb][v] = fmaf(s[jb], (float)P[v], acc[ib][jb][v]);
                }
        }
    };
    // step s (ring slot J = s % 4): its stage is in LDS buffer J % 2; the slot reloads stage
    // s + 4; stage s + 1 (loaded three steps ago) is staged into the other buffer
    auto step = [&](int s, auto jc, Stage &Rcur, Stage &Rnext) {
        constexpr int J = decltype(jc)::value;
        gload(s + 4, Rcur);
        lstore(IC<(J + 1) % 2>{}, Rnext);
        mfmas(IC<J % 2>{});
        __syncthreads();
    };
    // nk = K / 64 is a multiple of 4 (K is a multiple of 256): whole ring turns only
    for (int s = 0; s < nk; s += 4) {
        step(s, IC<0>{}, R0, R1);
        step(s + 1, IC<1>{}, R1, R2);
        step(s + 2, IC<2>{}, R2, R3);
        step(s + 3, IC<3>{}, R3, R0);
    }

    // ---- epilogue: lane holds column j = l32 (weight row), tokens 8(v/4) + 4 half + v%4
#pragma unroll
    for (int jb = 0; jb < JB; jb++) {
        const int64_t r = n0 + wn * (BN / 2) + jb * 32 + l32;
        if (r >= N) continue;
        const float rs_ = a.s_ch[r] * s_cb;
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t m = m0 + wm * 64 + ib * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                if (m < M) {
                    const float val = (acc[ib][jb][v] * rs_) * a.s_x[m];
                    if (a.y_bf16)
                        static_cast<uint16_t *>(a.y)[m * N + r] = f32_to_bf16_rne(val);
                    else
                        static_cast<float *>(a.y)[m * N + r] = val;
                }
            }
    }
}

}  // namespace

hipError_t launch_gemm_i8_fold(const LinearArgs &a, hipStream_t stream) {
    const int64_t tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    hipLaunchKernelGGL(k_gemm_i8_fold, dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream, a, (int)tm,
                       (int)(tm * tn));
    return hipGetLastError();
}

}  // namespace w4a8
