// Kernel 3a: prefill GEMM on int8 MFMA with the per-16 group scales folded into the
// exact int32 partial sums.
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
// Tile: 128 tokens x 128 rows per 256-thread workgroup (2 x 2 waves of 64 x 64), K steps of
// 64 (four groups) staged through double-buffered LDS.  Within every 8-wide K chunk the
// MFMA slot order is (0, 2, 4, 6, 1, 3, 5, 7): the activation tile is stored in that order
// so that a packed dword decodes with plain nibble masks (low nibbles = even k).
// Nibble -> int8 decode is a 16-entry byte table in four registers read with v_perm.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int int16v __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
// Padded LDS row strides: 72 B per activation row and 36 B per packed row put the 32 rows
// that one fragment read touches on distinct banks (LDS has 32 four-byte banks).
constexpr int kXRow = BK + 8, kPRow = BK / 2 + 4;

struct CbI8 {
    uint32_t t[4];  // cb_i8[0..15] as bytes
};

__device__ __forceinline__ uint32_t lookup4(const CbI8 &c, uint32_t idx4) {
    const uint32_t sel = idx4 & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(c.t[1], c.t[0], sel);
    const uint32_t hi = __builtin_amdgcn_perm(c.t[3], c.t[2], sel);
    const uint32_t msel = ((idx4 >> 3) & 0x01010101u) | 0x0C0C0C0Cu;  // 0x0C -> 0x00, 0x0D -> 0xFF
    const uint32_t mask = __builtin_amdgcn_perm(0u, 0u, msel);
    return (mask & hi) | (~mask & lo);
}

// 8 nibbles (k = 0..7 of a chunk) -> 8 int8 in slot order (0, 2, 4, 6, 1, 3, 5, 7).
__device__ __forceinline__ long decode8(const CbI8 &c, uint32_t w) {
    const uint32_t even = lookup4(c, w & 0x0F0F0F0Fu);
    const uint32_t odd = lookup4(c, (w >> 4) & 0x0F0F0F0Fu);
    return (long)(((uint64_t)odd << 32) | even);
}

// Activation bytes x0..x7 -> slot order (x0, x2, x4, x6, x1, x3, x5, x7).
__device__ __forceinline__ uint2 slot_order(uint32_t d0, uint32_t d1) {
    return make_uint2(__builtin_amdgcn_perm(d1, d0, 0x06040200u),
                      __builtin_amdgcn_perm(d1, d0, 0x07050301u));
}

__global__ __launch_bounds__(kThreads) void k_gemm_i8(LinearArgs a) {
    __shared__ __align__(16) uint8_t xs[2][BM * kXRow];
    __shared__ __align__(16) uint8_t ps[2][BN * kPRow];
    __shared__ __align__(16) uint8_t ss[2][BN * BK / kGroup];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

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
        for (int b = 0; b < 4; b++) {
            const int q = (s_cb > 0.0f) ? (int)rintf(a.cb[4 * w + b] / s_cb) : 0;
            v |= ((uint32_t)q & 0xFFu) << (8 * b);
        }
        cbt.t[w] = v;
    }

    // global -> register staging assignment (rows past M or N read row 0 and are zeroed)
    const int xr = tid >> 1, xh = tid & 1;      // x: row xr, 32 bytes at 32*xh
    const int pr = tid >> 1, ph = tid & 1;      // packed: row pr, 16 bytes at 16*ph
    const bool xvalid = m0 + xr < M, pvalid = n0 + pr < N;
    const bool svalid = tid < BN && n0 + tid < N;
    const uint4 *xsrc = reinterpret_cast<const uint4 *>(a.x_q + (xvalid ? (m0 + xr) * K : 0) + 32 * xh);
    const uint4 *psrc = reinterpret_cast<const uint4 *>(a.packed + (pvalid ? (n0 + pr) * (K / 2) : 0) + 16 * ph);
    const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(a.s_rel + (svalid ? (n0 + tid) * (K / kGroup) : 0));
    const uint32_t xmask = xvalid ? 0xFFFFFFFFu : 0u, pmask = pvalid ? 0xFFFFFFFFu : 0u;
    const uint32_t smask = svalid ? 0xFFFFFFFFu : 0u;
    uint8_t *xdst0 = &xs[0][xr * kXRow + 32 * xh];
    uint8_t *pdst0 = &ps[0][pr * kPRow + 16 * ph];
    uint8_t *sdst0 = &ss[0][(tid & (BN - 1)) * 4];
    constexpr int xbuf = BM * kXRow, pbuf = BN * kPRow, sbuf = BN * BK / kGroup;

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int nk = (int)(K / BK);
    uint4 rx0 = xsrc[0], rx1 = xsrc[1], rp = psrc[0];
    uint32_t rs = ssrc[0];
#define W4A8_STAGE_STORE(buf)                                                                   \
    do {                                                                                        \
        const uint2 o0 = slot_order(rx0.x & xmask, rx0.y & xmask);                              \
        const uint2 o1 = slot_order(rx0.z & xmask, rx0.w & xmask);                              \
        const uint2 o2 = slot_order(rx1.x & xmask, rx1.y & xmask);                              \
        const uint2 o3 = slot_order(rx1.z & xmask, rx1.w & xmask);                              \
        uint2 *dx = reinterpret_cast<uint2 *>(xdst0 + (buf) * xbuf);  /* 8-B aligned rows */   \
        dx[0] = o0; dx[1] = o1; dx[2] = o2; dx[3] = o3;                                         \
        uint32_t *dp = reinterpret_cast<uint32_t *>(pdst0 + (buf) * pbuf); /* 4-B aligned */    \
        dp[0] = rp.x & pmask; dp[1] = rp.y & pmask; dp[2] = rp.z & pmask; dp[3] = rp.w & pmask;  \
        if (tid < BN) *reinterpret_cast<uint32_t *>(sdst0 + (buf) * sbuf) = rs & smask;          \
    } while (0)
    W4A8_STAGE_STORE(0);
    __syncthreads();
    const int half = lane >> 5, l32 = lane & 31;
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            const int64_t k1 = (int64_t)(kt + 1) * BK;
            rx0 = xsrc[k1 / 16];
            rx1 = xsrc[k1 / 16 + 1];
            rp = psrc[k1 / 32];
            rs = ssrc[k1 / 64];
        }
        // rolled on purpose: each group's four MFMA results are folded before the next
        // group's MFMAs issue, so only 64 partials are live at a time
#pragma unroll 1
        for (int g = 0; g < BK / kGroup; g++) {
            long A[2], B[2];
            float s[2];
#pragma unroll
            for (int ib = 0; ib < 2; ib++) {
                const int row = wm * 64 + ib * 32 + l32;
                A[ib] = *reinterpret_cast<const long *>(&xs[buf][row * kXRow + g * kGroup + 8 * half]);
            }
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
                const int row = wn * 64 + jb * 32 + l32;
                const uint32_t w = *reinterpret_cast<const uint32_t *>(&ps[buf][row * kPRow + g * 8 + 4 * half]);
                B[jb] = decode8(cbt, w);
                s[jb] = e4m3_to_f32(ss[buf][row * 4 + g]);
            }
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
#pragma unroll
                for (int jb = 0; jb < 2; jb++) {
                    const int16v zero = {};
                    const int16v P = __builtin_amdgcn_mfma_i32_32x32x16_i8(A[ib], B[jb], zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 16; v++) acc[ib][jb][v] = fmaf(s[jb], (float)P[v], acc[ib][jb][v]);
                }
        }
        if (kt + 1 < nk) W4A8_STAGE_STORE(buf ^ 1);
        __syncthreads();
    }

#undef W4A8_STAGE_STORE

    // epilogue: lane holds column j = l32 (weight row) and rows i = 8(v/4) + 4 half + v%4
#pragma unroll
    for (int jb = 0; jb < 2; jb++) {
        const int64_t r = n0 + wn * 64 + jb * 32 + l32;
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

hipError_t launch_gemm_i8(const LinearArgs &a, hipStream_t stream) {
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(k_gemm_i8, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a8
