// Kernel 3: prefill GEMM on f16 MFMA over weights decoded once per tile, with the per-16
// group scale applied to each decoded weight.
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", sections "Format" and "Why this
// exists": 4-bit indices into a per-tensor 16-level codebook, an e4m3 scale per 16 values
// and an fp32 scale per output row, executed on the int8 GEMM path with a codebook
// dequantisation step on top.
//
// Two forms of the codebook, one skeleton (template flag I8):
//  * fp16 codebook (the automatic prefill route): w16 = fp16(s16 * cb16[idx]) with
//    cb16 = fp16(cb / 2^ex) (max |cb| = f 2^ex, f in [0.5, 1)) and s16 = s_rel * 2^7 (exact:
//    an e4m3 value times a power of two; every finite e4m3 magnitude, 2^-9 to 448, lands in
//    [2^-2, 57344], so s16 and s16 * cb16 stay below the fp16 maximum 65504).  Two fp16
//    roundings give at most ~2^-10 relative error per weight, inside the layer's
//    4e-3 * sum |x w| bound by construction; the 2^7 keeps products of small scales and
//    levels down to 2^-12 out of the fp16 subnormal range.
//      y[m, r] = acc * 2^(ex - 7) * s_channel[r] * s_x[m].
//  * int8 codebook (the int8 route): cb_i8 = rint(cb / s_cb), s_cb = max|cb| / 127, and
//    w16 = cb_i8[idx] * s_rel, which fp16 holds exactly: |cb_i8| <= 127 (7 bits) times an
//    e4m3 value (4 significant bits) has at most 11 significant bits, and the magnitudes run
//    from 2^-9 to 127 * 448 = 56896, inside fp16's normal range.  Every product x_q * w16 is
//    then exact in fp32 (8 + 11 bits), so each group's 16 products are exactly
//    s_rel * sum x_q * cb_i8 -- the per-16 partial with its group scale folded in -- and the
//    fp32 MFMA accumulation adds them up: the fold costs no vector-ALU work at all.
//      y[m, r] = acc * s_cb * s_channel[r] * s_x[m].
// x_q is exact in fp16.  With the group scale inside the weight, every group accumulates
// into the same fp32 MFMA accumulator.
//
// Tile (prefill): 256 tokens x 192 weight rows per 512-thread workgroup, one workgroup per
// CU (the 192-row tile divides both MLP shapes into nearly whole rounds of 256 tiles).  Waves
// 4 (tokens) x 2 (rows), each 64 x 96 = 2 x 3 fragments of v_mfma_f32_32x32x16_f16.  K
// advances in stages of 64, double-buffered through LDS; the global loads run four stages
// ahead in a ring of register stages, so a stage is decoded three steps after its loads
// were issued:
//  * activations: int8 -> fp16 once per stage (exact, v_perm onto 0x6400 then one packed
//    subtract) into [token][64 + 8 pad] rows;
//  * weights: decoded once per stage by the whole workgroup -- a packed byte indexes a
//    256-entry LDS table of fp16 pairs (level[low nibble], level[high nibble]), one packed
//    multiply applies the group scale -- into [row][64 + 8 pad] rows, so the MFMA loop
//    reads plain fp16 fragments for both operands.
// The 144-byte LDS rows put the 16 rows one 16-lane phase of a 16-byte fragment read
// touches on 16 distinct 16-byte bank quads of the 64 banks.  Tiles are numbered so that
// each XCD works through a contiguous run, token tiles fastest: the workgroups resident on
// one XCD share weight and activation stages through its L2.
#include <type_traits>

#include "e4m3_pair.h"
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int kPitch = BK + 8;                 // fp16 per LDS row (144 B)

// Tile configurations: BM tokens x BN weight rows per workgroup, WM x WN waves, each wave
// (BM / WM) x (BN / WN) as 32 x 32 fragments.  Every configuration accumulates each output
// over the same k order with the same MFMA, so they give identical results; the prefill one
// (256 x 192, 8 waves) suits many tokens, the small ones give a few dozen tokens enough
// workgroups for every CU.
template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int IB = BM / WM / 32, JB = BN / WN / 32;   // 32 x 32 fragments per wave
    static constexpr int kXStage = BM * kPitch, kBStage = BN * kPitch;
    static_assert(IB >= 1 && JB >= 1 && BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
    static_assert(2 * BM <= kThreads && 2 * BN <= kThreads && (2 * BN) % 64 == 0, "staging roles");
};
using CfgPrefill = Cfg<256, 192, 4, 2>;
using CfgSmall = Cfg<64, 64, 2, 2>;
using CfgTiny = Cfg<32, 64, 1, 2>;

// four int8 -> four fp16 (exact): bytes b ^ 0x80 under the fp16 exponent of 1024 give
// 1024 + b + 128; subtracting 1152 leaves b
__device__ __forceinline__ uint2 i8x4_to_f16x4(uint32_t v) {
    const uint32_t t = v ^ 0x80808080u;
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const half2_t lo = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, t, 0x04010400u)) - off;
    const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, t, 0x04030402u)) - off;
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

struct Stage {
    uint4 x0, x1;   // 32 activation bytes of token xr
    uint4 p;        // 32 packed indices of weight row pr (two groups)
    uint32_t s;     // the row's four e4m3 group scales of the stage
};

template <int J>
using IC = std::integral_constant<int, J>;

template <class C, bool I8>
__global__ __launch_bounds__(C::kThreads) void k_gemm_dec(LinearArgs a, int tiles_m, int tiles) {
    constexpr int BM = C::BM, BN = C::BN, IB = C::IB, JB = C::JB;
    constexpr int kXStage = C::kXStage, kBStage = C::kBStage;
    __shared__ __align__(16) _Float16 xs[2][kXStage];
    __shared__ __align__(16) _Float16 bs[2][kBStage];
    __shared__ uint32_t tab[256];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t M = a.M, N = a.N, K = a.K;

    // consecutive workgroups go to consecutive XCDs: XCD x takes the contiguous tile run
    // starting at x*q + min(x, rem)
    const int b = blockIdx.x, q = tiles / 8, rem = tiles % 8, xcd = b % 8, slot = b / 8;
    const int t = xcd * q + min(xcd, rem) + slot;
    const int64_t m0 = (int64_t)(t % tiles_m) * BM, n0 = (int64_t)(t / tiles_m) * BN;

    // ---- codebook pair table, entry e = (level[e & 15], level[e >> 4]): cb16 = fp16(cb / 2^ex),
    // or the integers cb_i8 = rint(cb / s_cb) (same fp32 arithmetic at every thread)
    float cmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kLevels; j++) cmax = fmaxf(cmax, fabsf(a.cb[j]));
    int ex = 0;
    if (cmax > 0.0f) frexpf(cmax, &ex);
    const float s_cb = cmax / 127.0f;
    auto level = [&](int j) {
        if constexpr (I8) return (s_cb > 0.0f) ? rintf(a.cb[j] / s_cb) : 0.0f;
        else return a.cb[j] * ldexpf(1.0f, -ex);
    };
    for (int e = tid; e < 256; e += C::kThreads)   // fewer than 256 threads: several entries each
        tab[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)level(e & 15)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)level(e >> 4)) << 16);

    // ---- staging roles: token xr, bytes [32 xh, 32 xh + 32) of a stage; weight row pr,
    // weights [32 ph, 32 ph + 32) (two groups).  Rows past M or N re-read the last valid row:
    // they feed only outputs that are never stored.  Threads past 2 BN load like the last
    // row's but decode nothing; threads past 2 BM load like the last token's and stage
    // nothing.
    const bool xdec = (tid >> 1) < BM;             // wave-uniform: 2 BM is a multiple of 64
    const int xr = xdec ? tid >> 1 : BM - 1, xh = tid & 1;
    const int pr0 = tid >> 1, ph = tid & 1;
    const bool pdec = pr0 < BN;                    // wave-uniform: 2 BN is a multiple of 64
    const int pr = pdec ? pr0 : BN - 1;
    const int8_t *xp = a.x_q + min<int64_t>(m0 + xr, M - 1) * K + 32 * xh;
    const int64_t wrow = min<int64_t>(n0 + pr, N - 1);
    const int8_t *pp = a.packed + wrow * (K / 2) + 16 * ph;
    // a row's group scales start 16-byte aligned (K / 16 is a multiple of 16); one dword
    // holds the stage's four
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(a.s_rel + wrow * (K / kGroup));
    const int sshift = 16 * ph;
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
    _Float16 *const xdst = &xs[0][xr * kPitch + 32 * xh];
    _Float16 *const bdst = &bs[0][pr * kPitch + 32 * ph];
    auto lstore = [&](auto bufc, const Stage &st) {
        constexpr int buf = decltype(bufc)::value;
        const uint32_t xw[8] = {st.x0.x, st.x0.y, st.x0.z, st.x0.w, st.x1.x, st.x1.y, st.x1.z, st.x1.w};
        if (xdec) {
            uint4 *dx = reinterpret_cast<uint4 *>(xdst + buf * kXStage);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint2 c0 = i8x4_to_f16x4(xw[2 * i]), c1 = i8x4_to_f16x4(xw[2 * i + 1]);
                dx[i] = make_uint4(c0.x, c0.y, c1.x, c1.y);
            }
        }
        if (pdec) {
            const uint32_t sv = st.s >> sshift;
            constexpr float kPre = I8 ? 1.0f : 128.0f;  // exact: a power of two
            const uint32_t s2 = e4m3x2_to_f16x2(sv, kPre);
            const half2_t g0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, s2, 0x01000100u));
            const half2_t g1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, s2, 0x03020302u));
            const uint32_t pw[4] = {st.p.x, st.p.y, st.p.z, st.p.w};
            uint32_t o[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const half2_t pair = __builtin_bit_cast(half2_t, tab[(pw[i >> 2] >> (8 * (i & 3))) & 0xFFu]);
                o[i] = __builtin_bit_cast(uint32_t, pair * (i < 8 ? g0 : g1));
            }
            uint4 *db = reinterpret_cast<uint4 *>(bdst + buf * kBStage);
#pragma unroll
            for (int i = 0; i < 4; i++) db[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        }
    };

    float16_t acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; i++)
#pragma unroll
        for (int j = 0; j < JB; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    Stage R0, R1, R2, R3;
    gload(0, R0);
    gload(1, R1);
    gload(2, R2);
    gload(3, R3);
    __syncthreads();
    lstore(IC<0>{}, R0);
    __syncthreads();

    const int half = lane >> 5, l32 = lane & 31;
    const _Float16 *const xrd = &xs[0][(wm * (BM / C::WM) + l32) * kPitch + 8 * half];
    const _Float16 *const brd = &bs[0][(wn * (BN / C::WN) + l32) * kPitch + 8 * half];

    auto mfmas = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int g = 0; g < BK / 16; g++) {
            half8_t A[IB], B[JB];
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
                A[ib] = *reinterpret_cast<const half8_t *>(xrd + buf * kXStage + ib * 32 * kPitch + g * 16);
#pragma unroll
            for (int jb = 0; jb < JB; jb++)
                B[jb] = *reinterpret_cast<const half8_t *>(brd + buf * kBStage + jb * 32 * kPitch + g * 16);
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
#pragma unroll
                for (int jb = 0; jb < JB; jb++)
                    acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[ib], B[jb], acc[ib][jb], 0, 0, 0);
        }
    };
    // step s (ring slot J = s % 4): its stage is in LDS buffer J % 2; the slot reloads stage
    // s + 4; stage s + 1 (loaded three steps ago) is decoded into the other buffer
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
    const float scale = I8 ? s_cb : ldexpf(1.0f, ex - 7);
#pragma unroll
    for (int jb = 0; jb < JB; jb++) {
        const int64_t r = n0 + wn * (BN / C::WN) + jb * 32 + l32;
        if (r >= N) continue;
        const float rsc = a.s_ch[r] * scale;
#pragma unroll
        for (int ib = 0; ib < IB; ib++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t m = m0 + wm * (BM / C::WM) + ib * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                if (m < M) {
                    const float val = (acc[ib][jb][v] * rsc) * a.s_x[m];
                    if (a.y_bf16)
                        static_cast<uint16_t *>(a.y)[m * N + r] = f32_to_bf16_rne(val);
                    else
                        static_cast<float *>(a.y)[m * N + r] = val;
                }
            }
    }
}

template <class C, bool I8>
hipError_t launch_cfg(const LinearArgs &a, hipStream_t stream) {
    const int64_t tm = (a.M + C::BM - 1) / C::BM, tn = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL((k_gemm_dec<C, I8>), dim3((unsigned)(tm * tn)), dim3(C::kThreads), 0, stream, a, (int)tm,
                       (int)(tm * tn));
    return hipGetLastError();
}

template <bool I8>
hipError_t launch_form(const LinearArgs &a, hipStream_t stream) {
    if (a.M <= CfgTiny::BM) return launch_cfg<CfgTiny, I8>(a, stream);
    if (a.M <= CfgSmall::BM) return launch_cfg<CfgSmall, I8>(a, stream);
    return launch_cfg<CfgPrefill, I8>(a, stream);
}

}  // namespace

// The tile configuration by token count: the results do not depend on it.
hipError_t launch_gemm_f16(const LinearArgs &a, hipStream_t stream) { return launch_form<false>(a, stream); }
hipError_t launch_gemm_i8(const LinearArgs &a, hipStream_t stream) { return launch_form<true>(a, stream); }

bool gemm_dec_tiles_fit(int64_t M, int64_t N) {
    const int64_t bm = M <= CfgTiny::BM ? CfgTiny::BM : (M <= CfgSmall::BM ? CfgSmall::BM : CfgPrefill::BM);
    const int64_t bn = M <= CfgSmall::BM ? CfgSmall::BN : CfgPrefill::BN;
    return ((M + bm - 1) / bm) * ((N + bn - 1) / bn) <= (int64_t(1) << 31) - 1;
}

}  // namespace w4a8
