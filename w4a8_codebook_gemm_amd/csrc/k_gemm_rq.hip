// Kernel 3c: prefill GEMM on requantised int8 weights.
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", sections "Why this exists"
// and "Format": the W4A8 layer runs on the same int8 GEMM path as INT8 and adds a
// codebook dequantisation step; int4 indices, a per-tensor 16-level codebook, an e4m3
// scale per 16 values and an fp32 scale per output row.
//
// The second int8 reading of that step.  Each weight is decoded with its group scale and
// rounded to int8 on one per-tensor step s_cb = max|cb| / 127:
//   q[r, k] = rint(fl(dec(s_rel[r, g]) * cb[idx[r, k]]) / s_cb), clamped to +-127
// (0 for the two NaN codes), so one int32 sum covers the whole row and the scales enter
// once, in the epilogue:
//   y[m, r] = ((float)sum_k x_q[m, k] q[r, k] * (s_channel[r] * s_cb)) * s_x[m].
// The sum is exact in int32 for K <= 131072.  The group scale takes only 256 values, so
// each workgroup first fills the table t[code][index] (4 KB of LDS) with the same fp32
// arithmetic; a group of 16 then decodes with one 16-byte table read and byte-permute
// lookups.  The result differs from the exact product by the rounding of each weight to
// the step (at most s_cb / 2 in units of the row scale when every |dec(s_rel)| <= 1).
//
// No group boundary falls inside the integer sum, so the kernel runs the full-rate
// v_mfma_i32_32x32x32_i8.  Tile and schedule follow the W8A8 comparator's GEMM: 256 tokens
// x 192 weight rows per 512-thread workgroup (4 x 2 waves of 64 x 96), one workgroup per
// CU, 64-byte K stages double-buffered through LDS with the global loads four stages ahead
// in a ring of register stages, int32 accumulation over all of K.  Per stage each thread
// copies 32 activation bytes and decodes one group of 16 weights (8 packed bytes and one
// scale byte; threads < 256 a second group of row + 128), which spreads the decode evenly
// over the four SIMDs.  Tiles are numbered so that each XCD works through a contiguous run
// of them, token tiles fastest.
#include <type_traits>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));

constexpr int GM = 256, GN = 192, GK = 64;  // tile: tokens x weight rows x K per stage
constexpr int kThreads = 512;
constexpr int GJB = GN / 64;                // 32-row weight blocks per wave
// 80-byte LDS rows: the 16 rows one 16-lane phase of a 16-byte fragment read touches start
// at distinct multiples of 16 bytes modulo 256, i.e. on disjoint bank quads
constexpr int kPitch = GK + 16;
constexpr int kXSt = GM * kPitch, kWSt = GN * kPitch;
constexpr int kCodes = 256;

struct RStage {
    int4v x0, x1;      // 32 activation bytes of token xr
    uint2 p0, p1;      // 16 packed indices (one group) of rows wr and wr + 128
    uint32_t s0, s1;   // their e4m3 group scales
};

template <int J>
using RIC = std::integral_constant<int, J>;

// two waves per SIMD: the accumulators and the register ring need up to 256 registers
__global__ __launch_bounds__(kThreads, 1) void k_gemm_rq(LinearArgs a, int tiles_m, int tiles) {
    __shared__ __align__(16) int8_t xs[2][kXSt];
    __shared__ __align__(16) int8_t ws[2][kWSt];
    __shared__ __align__(16) uint8_t tab[kCodes * kLevels];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;

    const int b = blockIdx.x, q = tiles / 8, rem = tiles % 8, xcd = b % 8, slot = b / 8;
    const int t = xcd * q + min(xcd, rem) + slot;
    const int64_t m0 = (int64_t)(t % tiles_m) * GM, n0 = (int64_t)(t / tiles_m) * GN;

    // ---- staging roles (every load is issued before the table is built)
    static_assert(GN > 128 && GN <= 256 && kThreads == 512, "weight staging covers 128 + (GN - 128) rows");
    const int xr = tid >> 1, xh = tid & 1;
    const int wr = tid >> 2, wq = tid & 3;
    const bool w1st = wr < GN - 128;               // wave-uniform: 4 (GN - 128) is a multiple of 64
    const int64_t r0 = min<int64_t>(n0 + wr, N - 1);
    const int64_t r1 = min<int64_t>(n0 + (w1st ? 128 + wr : GN - 1), N - 1);
    const int8_t *xp = a.x_q + min<int64_t>(m0 + xr, M - 1) * K + 32 * xh;
    const int8_t *pp0 = a.packed + r0 * (K / 2) + 8 * wq;
    const int8_t *pp1 = a.packed + r1 * (K / 2) + 8 * wq;
    const uint8_t *sp0 = a.s_rel + r0 * (K / kGroup) + wq;
    const uint8_t *sp1 = a.s_rel + r1 * (K / kGroup) + wq;
    const int nk = (int)(K / GK);

    // every stage's loads are issued unconditionally (stages past the end re-read the last
    // one) so that the in-order load counter lets a store wait for its own stage only
    auto gload = [&](int kt, RStage &st) {
        const int64_t k = kt < nk ? kt : nk - 1;
        st.x0 = *reinterpret_cast<const int4v *>(xp + k * GK);
        st.x1 = *reinterpret_cast<const int4v *>(xp + k * GK + 16);
        st.p0 = *reinterpret_cast<const uint2 *>(pp0 + k * (GK / 2));
        st.p1 = *reinterpret_cast<const uint2 *>(pp1 + k * (GK / 2));
        st.s0 = sp0[k * (GK / kGroup)];
        st.s1 = sp1[k * (GK / kGroup)];
    };

    RStage R0, R1, R2, R3;
    gload(0, R0);
    gload(1, R1);
    gload(2, R2);
    gload(3, R3);

    // ---- the requantised level table: thread tid fills code tid / 2, levels 8 (tid % 2) ..
    float cmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kLevels; j++) cmax = fmaxf(cmax, fabsf(a.cb[j]));
    const float s_cb = cmax / 127.0f;
    {
        const int c = tid >> 1, j0 = 8 * (tid & 1);
        // gfx950's v_cvt_f32_fp8 decodes OCP E4M3FN exactly
        const float d = __builtin_amdgcn_cvt_f32_fp8(c, 0);
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
            const float prod = d * a.cb[j0 + jj];
            const float v = prod / s_cb;
            int qv = 0;
            if ((c & 0x7F) != 0x7F && v == v) qv = (int)fminf(fmaxf(rintf(v), -127.0f), 127.0f);
            w[jj >> 2] |= ((uint32_t)qv & 0xFFu) << (8 * (jj & 3));
        }
        *reinterpret_cast<uint2 *>(&tab[c * kLevels + j0]) = make_uint2(w[0], w[1]);
    }
    __syncthreads();

    int8_t *const xdst = &xs[0][xr * kPitch + 32 * xh];
    int8_t *const wdst = &ws[0][wr * kPitch + 16 * wq];   // row wr; row wr + 128 is 128 rows on
    auto decode16 = [&](uint32_t code, uint2 p) {
        const uint4 tv = *reinterpret_cast<const uint4 *>(&tab[code * kLevels]);
        const CbI8 c{{tv.x, tv.y, tv.z, tv.w}};
        const uint2 lo = decode8(c, p.x), hi = decode8(c, p.y);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    auto lstore = [&](auto bufc, const RStage &st) {
        constexpr int buf = decltype(bufc)::value;
        int4v *dx = reinterpret_cast<int4v *>(xdst + buf * kXSt);
        dx[0] = st.x0;
        dx[1] = st.x1;
        *reinterpret_cast<uint4 *>(wdst + buf * kWSt) = decode16(st.s0, st.p0);
        if (w1st) *reinterpret_cast<uint4 *>(wdst + buf * kWSt + 128 * kPitch) = decode16(st.s1, st.p1);
    };

    int16v acc[2][GJB];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < GJB; j++) acc[i][j] = int16v{};

    lstore(RIC<0>{}, R0);
    __syncthreads();

    const int half = lane >> 5, l32 = lane & 31;
    const int8_t *const xrd = &xs[0][(wm * 64 + l32) * kPitch + 16 * half];
    const int8_t *const wrd = &ws[0][(wn * (GN / 2) + l32) * kPitch + 16 * half];
    auto mfmas = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int s = 0; s < GK / 32; s++) {
            int4v A[2], B[GJB];
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
                A[ib] = *reinterpret_cast<const int4v *>(xrd + buf * kXSt + ib * 32 * kPitch + s * 32);
#pragma unroll
            for (int jb = 0; jb < GJB; jb++)
                B[jb] = *reinterpret_cast<const int4v *>(wrd + buf * kWSt + jb * 32 * kPitch + s * 32);
            // A and B lanes carry the same 16 k of the 32-wide step, so the product is the
            // full sum over the step whatever order the unit takes them in
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
#pragma unroll
                for (int jb = 0; jb < GJB; jb++)
                    acc[ib][jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ib], B[jb], acc[ib][jb], 0, 0, 0);
        }
    };
    // step s (ring slot J = s % 4): its stage is in LDS buffer J % 2; the slot reloads stage
    // s + 4; stage s + 1 (loaded three steps ago) is decoded into the other buffer
    auto step = [&](int s, auto jc, RStage &Rcur, RStage &Rnext) {
        constexpr int J = decltype(jc)::value;
        gload(s + 4, Rcur);
        lstore(RIC<(J + 1) % 2>{}, Rnext);
        mfmas(RIC<J % 2>{});
        __syncthreads();
    };
    // nk = K / 64 is a multiple of 4 (K is a multiple of 256): whole ring turns only
    for (int s = 0; s < nk; s += 4) {
        step(s, RIC<0>{}, R0, R1);
        step(s + 1, RIC<1>{}, R1, R2);
        step(s + 2, RIC<2>{}, R2, R3);
        step(s + 3, RIC<3>{}, R3, R0);
    }

    // lane holds weight row j = l32 of each 32 x 32 block and tokens 8(v/4) + 4 half + v%4
#pragma unroll
    for (int jb = 0; jb < GJB; jb++) {
        const int64_t r = n0 + wn * (GN / 2) + jb * 32 + l32;
        if (r >= N) continue;
        const float sw = a.s_ch[r] * s_cb;
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

bool gemm_rq_supported(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + GM - 1) / GM) * ((N + GN - 1) / GN);
    return K <= 131072 && tiles <= (int64_t(1) << 31) - 1;
}

hipError_t launch_gemm_rq(const LinearArgs &a, hipStream_t stream) {
    const int64_t tm = (a.M + GM - 1) / GM, tn = (a.N + GN - 1) / GN;
    hipLaunchKernelGGL(k_gemm_rq, dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream, a, (int)tm,
                       (int)(tm * tn));
    return hipGetLastError();
}

}  // namespace w4a8
