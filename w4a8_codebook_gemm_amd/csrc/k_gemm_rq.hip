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
// v_mfma_i32_32x32x32_i8.  Tile: 256 tokens x 192 weight rows per 512-thread workgroup
// (4 x 2 waves of 64 x 96), one workgroup per CU, int32 accumulation over all of K.
//  * K advances in stages of 128, double-buffered through LDS in 144-byte rows (the 16
//    rows one phase of a 16-byte fragment read touches start on distinct bank quads).
//  * Every global load covers whole 128-byte lines: eight lanes per row, 16 activation
//    bytes or one group (8 packed bytes and its scale byte) per lane, eight rows per load.
//    Each thread copies four activation chunks and decodes three groups per stage, the
//    same for every wave.  A stage's loads are issued one stage ahead into a ring of two
//    register stages.
//  * Each stage is scheduled by hand: the fragments of 32-k step t + 1 are read while step
//    t's six MFMAs run, and the next stage's decode (table read, lookups, LDS store) is
//    spread between them, so neither the LDS latency nor the decode stalls the MFMA issue.
// Tiles are numbered so that each XCD works through a contiguous run of them, token tiles
// fastest.

#include <type_traits>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));

constexpr int GM = 256, GN = 192, GK = 128;  // tile: tokens x weight rows x K per stage
constexpr int kThreads = 512;
constexpr int GJB = GN / 64;                 // 32-row weight blocks per wave
constexpr int kPitch = GK + 16;
constexpr int kXSt = GM * kPitch, kWSt = GN * kPitch;
constexpr int XJ = GM / 64, WJ = GN / 64;    // staged rows per thread: 4 activation, 3 weight
constexpr int kCodes = 256;

struct RStage {
    int4v x[XJ];      // 16 activation bytes of rows sr + 64 j
    uint2 p[WJ];      // the packed group (16 indices) of weight rows sr + 64 j
    uint32_t s[WJ];   // their e4m3 group scales
};

struct Frag {
    int4v A[2], B[GJB];
};

template <int J>
using RIC = std::integral_constant<int, J>;

// two waves per SIMD: the accumulators, two fragment sets and the register ring
__global__ __launch_bounds__(kThreads, 1) void k_gemm_rq(LinearArgs a, int tiles_m, int tiles) {
    __shared__ __align__(16) int8_t xs[2 * kXSt];
    __shared__ __align__(16) int8_t ws[2 * kWSt];
    __shared__ __align__(16) uint8_t tab[kCodes * kLevels];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;

    const int b = blockIdx.x, q = tiles / 8, rem = tiles % 8, xcd = b % 8, slot = b / 8;
    const int t = xcd * q + min(xcd, rem) + slot;
    const int64_t m0 = (int64_t)(t % tiles_m) * GM, n0 = (int64_t)(t / tiles_m) * GN;

    // ---- staging roles: rows sr + 64 j, 16-byte chunk / group sc of the stage.  Rows past
    // M or N re-read the last valid row: they feed only outputs that are never stored.
    const int sr = tid >> 3, sc = tid & 7;
    const int8_t *xp[XJ];
    const int8_t *pp[WJ];
    const uint8_t *spp[WJ];
#pragma unroll
    for (int j = 0; j < XJ; j++) xp[j] = a.x_q + min<int64_t>(m0 + sr + 64 * j, M - 1) * K + 16 * sc;
#pragma unroll
    for (int j = 0; j < WJ; j++) {
        const int64_t r = min<int64_t>(n0 + sr + 64 * j, N - 1);
        pp[j] = a.packed + r * (K / 2) + 8 * sc;
        spp[j] = a.s_rel + r * (K / kGroup) + sc;
    }
    const int nk = (int)(K / GK);  // even: K is a multiple of 256

    // every stage's loads are issued unconditionally (stages past the end re-read the last
    // one) so that the in-order load counter lets a decode wait for its own stage only
    auto gload = [&](int kt, RStage &st) {
        const int64_t k = kt < nk ? kt : nk - 1;
#pragma unroll
        for (int j = 0; j < XJ; j++) st.x[j] = *reinterpret_cast<const int4v *>(xp[j] + k * GK);
#pragma unroll
        for (int j = 0; j < WJ; j++) st.p[j] = *reinterpret_cast<const uint2 *>(pp[j] + k * (GK / 2));
#pragma unroll
        for (int j = 0; j < WJ; j++) st.s[j] = spp[j][k * (GK / kGroup)];
    };
    RStage R0, R1;
    gload(0, R0);
    gload(1, R1);

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

    auto tabrd = [&](uint32_t code) { return *reinterpret_cast<const uint4 *>(&tab[code * kLevels]); };
    auto decode16 = [&](uint4 tv, uint2 p) {
        const CbI8 c{{tv.x, tv.y, tv.z, tv.w}};
        const uint2 lo = decode8(c, p.x), hi = decode8(c, p.y);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    auto xstore = [&](int buf, const RStage &st) {
#pragma unroll
        for (int j = 0; j < XJ; j++)
            *reinterpret_cast<int4v *>(&xs[buf * kXSt + (sr + 64 * j) * kPitch + 16 * sc]) = st.x[j];
    };
    auto wstore = [&](int buf, int j, uint4 v) {
        *reinterpret_cast<uint4 *>(&ws[buf * kWSt + (sr + 64 * j) * kPitch + 16 * sc]) = v;
    };

    int16v acc[2][GJB];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < GJB; j++) acc[i][j] = int16v{};

    xstore(0, R0);
#pragma unroll
    for (int j = 0; j < WJ; j++) wstore(0, j, decode16(tabrd(R0.s[j]), R0.p[j]));
    __syncthreads();

    const int half = lane >> 5, l32 = lane & 31;
    const int8_t *const xrd = &xs[(wm * 64 + l32) * kPitch + 16 * half];
    const int8_t *const wrd = &ws[(wn * (GN / 2) + l32) * kPitch + 16 * half];
    // A and B lanes carry the same 16 k of a 32-wide step, so the product is the full sum
    // over the step whatever order the unit takes them in
    auto frag = [&](int buf, int s, Frag &f) {
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
            f.A[ib] = *reinterpret_cast<const int4v *>(xrd + buf * kXSt + ib * 32 * kPitch + s * 32);
#pragma unroll
        for (int jb = 0; jb < GJB; jb++)
            f.B[jb] = *reinterpret_cast<const int4v *>(wrd + buf * kWSt + jb * 32 * kPitch + s * 32);
    };
    auto mma3 = [&](const Frag &f, int ib) {
#pragma unroll
        for (int jb = 0; jb < GJB; jb++)
            acc[ib][jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.A[ib], f.B[jb], acc[ib][jb], 0, 0, 0);
    };
    // One stage: the MFMAs of buffer cur (four 32-k steps) while stage data nx is staged
    // into buffer cur ^ 1.  The scheduling barriers keep this issue order: the fragments of
    // step t + 1 and the table read of the next group go out before step t's MFMAs, and a
    // group's lookups sit between two halves of a step's MFMAs.
    auto stage = [&](auto curc, const RStage &nx) {
        constexpr int cur = decltype(curc)::value, oth = cur ^ 1;
        Frag F0, F1;
        frag(cur, 0, F0);
        __builtin_amdgcn_sched_barrier(0);
        uint4 tv = tabrd(nx.s[0]);
        __builtin_amdgcn_sched_barrier(0);
        xstore(oth, nx);
        frag(cur, 1, F1);
        __builtin_amdgcn_sched_barrier(0);
        mma3(F0, 0);
        const uint4 d0 = decode16(tv, nx.p[0]);
        mma3(F0, 1);
        __builtin_amdgcn_sched_barrier(0);
        wstore(oth, 0, d0);
        tv = tabrd(nx.s[1]);
        __builtin_amdgcn_sched_barrier(0);
        frag(cur, 2, F0);
        __builtin_amdgcn_sched_barrier(0);
        mma3(F1, 0);
        const uint4 d1 = decode16(tv, nx.p[1]);
        mma3(F1, 1);
        __builtin_amdgcn_sched_barrier(0);
        wstore(oth, 1, d1);
        tv = tabrd(nx.s[2]);
        __builtin_amdgcn_sched_barrier(0);
        frag(cur, 3, F1);
        __builtin_amdgcn_sched_barrier(0);
        mma3(F0, 0);
        const uint4 d2 = decode16(tv, nx.p[2]);
        mma3(F0, 1);
        __builtin_amdgcn_sched_barrier(0);
        wstore(oth, 2, d2);
        __builtin_amdgcn_sched_barrier(0);
        mma3(F1, 0);
        mma3(F1, 1);
    };
    // stage s is in LDS buffer s % 2 and stage s + 1 in ring slot (s + 1) % 2; the slot of
    // stage s (already staged) is reloaded with stage s + 2 first
    for (int s = 0; s < nk; s += 2) {
        gload(s + 2, R0);
        stage(RIC<0>{}, R1);
        __syncthreads();
        gload(s + 3, R1);
        stage(RIC<1>{}, R0);
        __syncthreads();
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
