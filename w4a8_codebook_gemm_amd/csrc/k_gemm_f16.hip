// Kernel 3b: prefill GEMM on f16 MFMA with the group scale folded into the decoded weight.
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", sections "Format" and "Why this
// exists": 4-bit indices into a per-tensor 16-level codebook, an e4m3 scale per 16 values
// and an fp32 scale per output row, executed on the GEMM path with a codebook
// dequantisation step on top.
//
// Each weight is decoded once per tile to fp16 w16 = fp16(s16 * cb16[idx]) with
// cb16 = fp16(cb / 2^ex) (max |cb| = f 2^ex, f in [0.5, 1)) and s16 = s_rel * 2^8 (exact:
// an e4m3 value times a power of two).  Two fp16 roundings give at most ~2^-10 relative
// error per weight, inside the layer's 4e-3 * sum |x w| bound by construction; the 2^8
// keeps products of small scales and levels out of the fp16 subnormal range.  x_q is exact
// in fp16.  With the group scale inside the weight, every group accumulates into the same
// fp32 MFMA accumulator: no per-group fold on the vector ALU.
//   y[m, r] = acc * 2^(ex - 8) * s_channel[r] * s_x[m].
//
// Tile: 128 tokens x 256 rows per 256-thread workgroup; waves 2 (tokens) x 2 (rows), each
// 64 x 128 = 2 x 4 fragments of v_mfma_f32_32x32x16_f16 (one 16-k group per MFMA).  K
// steps of 64 are staged through double-buffered LDS:
//  * activations as fp16, [token][64 + 8 pad] (16-B fragment reads spread over the banks);
//  * the fp16 codebook-pair table (256 packed-byte values x 32 columns, 256-B rows) as in
//    the decode GEMV: one v_perm address + one ds_read_b32 per packed byte;
//  * the packed indices and the fp16x2 group scales in the unused second half of every
//    table row, stored [k-slot][row] so that a fragment's 32 lanes read 32 consecutive
//    dwords.
#include <algorithm>
#include <type_traits>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kXRow = BK + 8;                      // fp16 per staged activation row (padded)
constexpr int kXTile = BM * kXRow;                 // fp16 per activation stage
constexpr int kTabBytes = 256 * 256;               // pair table rows of 256 B
// hole space (second 128 B of each table row): per stage 8 KiB packed + 4 KiB scales
constexpr int kPkBytes = BN * BK / 2;              // [8 k-slots][BN rows] dwords
constexpr int kSsBytes = BN * (BK / kGroup) * 4;   // [4 groups][BN rows] fp16x2
constexpr int kStageHole = kPkBytes + kSsBytes;

__device__ __forceinline__ uint32_t lds_u32(const char *base, uint32_t byte_addr) {
    return *reinterpret_cast<const uint32_t *>(base + byte_addr);
}

__global__ __launch_bounds__(kThreads) void k_gemm_f16(LinearArgs a) {
    __shared__ __align__(16) char tab[kTabBytes];                 // table + holes
    __shared__ __align__(16) _Float16 xs[2][kXTile];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

    // ---- staging assignment (rows past M or N read as zero via buffer bounds)
    const uint32_t rowbytes = (uint32_t)(K / 2), grpbytes = (uint32_t)(K / kGroup);
    const int64_t nvalid = std::min<int64_t>(BN, N - n0), mvalid = std::min<int64_t>(BM, M - m0);
    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.x_q + m0 * K), (short)0, (int)(mvalid * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.packed + n0 * rowbytes), (short)0, (int)(nvalid * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.s_rel + n0 * grpbytes), (short)0, (int)(nvalid * grpbytes), 0x00020000);
    const int xr = tid >> 1, xh = tid & 1;     // activations: token xr, 32 values at 32 xh
    const int pr = tid;                        // packed + scales: row pr (32 B + 4 codes)

    // ---- codebook pair table: cb16 = fp16(cb / 2^ex); entry e at e*256 + 4*column
    float cmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kLevels; j++) cmax = fmaxf(cmax, fabsf(a.cb[j]));
    int ex = 0;
    if (cmax > 0.0f) frexpf(cmax, &ex);
    const float inv = ldexpf(1.0f, -ex);
    {
        const int e0 = tid;  // 256 threads: one entry each, 32 columns
        const uint32_t v = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(a.cb[e0 & 15] * inv)) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(a.cb[e0 >> 4] * inv)) << 16);
        uint4 *row = reinterpret_cast<uint4 *>(tab + e0 * 256);
#pragma unroll
        for (int c = 0; c < 8; c++) row[c] = make_uint4(v, v, v, v);
    }

    // Global loads run two K steps ahead of their use, in two register sets: the loads for
    // step s are issued at the start of step s-2 and written to LDS at the end of step s-1.
    struct Stage {
        u32x4_t x0, x1, p0, p1;
        uint32_t s;
    };
    auto gload = [&](int64_t k0, Stage &st) {
        const uint32_t xo = (uint32_t)(xr * K + k0 + 32 * xh);
        st.x0 = __builtin_amdgcn_raw_buffer_load_b128(rs_x, xo, 0, 0);
        st.x1 = __builtin_amdgcn_raw_buffer_load_b128(rs_x, xo + 16, 0, 0);
        const uint32_t po = (uint32_t)(pr * rowbytes + k0 / 2);
        st.p0 = __builtin_amdgcn_raw_buffer_load_b128(rs_p, po, 0, 0);
        st.p1 = __builtin_amdgcn_raw_buffer_load_b128(rs_p, po + 16, 0, 0);
        st.s = __builtin_amdgcn_raw_buffer_load_b32(rs_s, (uint32_t)(pr * grpbytes + k0 / kGroup), 0, 0);
    };
    auto cvt2 = [](uint32_t v, int sh) {  // two int8 -> fp16x2 (exact)
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int8_t)((v >> sh) & 0xFF)) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int8_t)((v >> (sh + 8)) & 0xFF)) << 16);
    };
    // Hole space of stage b: k-slot s (= 2 g + h) of row r at dword (s * BN + r), then the
    // scales of group g of row r at dword (kPkBytes / 4 + g * BN + r).  A dword index d maps
    // to LDS byte (d / 32) * 256 + 128 + (d % 32) * 4.  Writer: row pr; readers: row
    // wn*128 + jb*32 + l32.  Both reduce to a per-lane base plus compile-time offsets.
    char *const st_base = tab + ((pr >> 5) << 8) + 128 + ((pr & 31) << 2);
    auto lstore = [&](int buf, const Stage &st) {
        uint4 *dx = reinterpret_cast<uint4 *>(&xs[buf][xr * kXRow + 32 * xh]);
        const uint32_t w[8] = {st.x0.x, st.x0.y, st.x0.z, st.x0.w, st.x1.x, st.x1.y, st.x1.z, st.x1.w};
#pragma unroll
        for (int q = 0; q < 4; q++)
            dx[q] = make_uint4(cvt2(w[2 * q], 0), cvt2(w[2 * q], 16), cvt2(w[2 * q + 1], 0), cvt2(w[2 * q + 1], 16));
        char *sb = st_base + buf * (2 * kStageHole);  // hole bytes map 128 -> 256
        const uint32_t p[8] = {st.p0.x, st.p0.y, st.p0.z, st.p0.w, st.p1.x, st.p1.y, st.p1.z, st.p1.w};
#pragma unroll
        for (int k = 0; k < 8; k++) *reinterpret_cast<uint32_t *>(sb + k * (BN / 32) * 256) = p[k];
        const float sv[4] = {__builtin_amdgcn_cvt_f32_fp8((int)st.s, 0), __builtin_amdgcn_cvt_f32_fp8((int)st.s, 1),
                             __builtin_amdgcn_cvt_f32_fp8((int)st.s, 2), __builtin_amdgcn_cvt_f32_fp8((int)st.s, 3)};
#pragma unroll
        for (int g = 0; g < 4; g++) {  // group scale as fp16x2, times 2^8
            const uint32_t h16 = __builtin_bit_cast(uint16_t, (_Float16)(sv[g] * 256.0f));
            *reinterpret_cast<uint32_t *>(sb + (kPkBytes / 128) * 256 + g * (BN / 32) * 256) = h16 | (h16 << 16);
        }
    };

    float16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int nk = (int)(K / BK);
    Stage R0, R1;  // register stages for even / odd K steps (compile-time selected)
    gload(0, R0);
    if (nk > 1) gload(BK, R1);
    lstore(0, R0);
    __syncthreads();
    const int half = lane >> 5, l32 = lane & 31;
    const uint32_t lanebase = (uint32_t)l32 * 4u;
    const char *rd_base = tab + ((wn * 128) >> 5) * 256 + 128 + l32 * 4 + half * (BN / 32) * 256;

    // one K step on LDS stage BUF, with R the register stage of this step's parity
    auto kstep = [&](int kt, auto bufc, Stage &Rcur, Stage &Rnext) {
        constexpr int buf = decltype(bufc)::value;
        if (kt + 2 < nk) gload((int64_t)(kt + 2) * BK, Rcur);
        const char *rb = rd_base + buf * (2 * kStageHole);
#pragma unroll
        for (int g = 0; g < BK / kGroup; g++) {
            half8_t A[2];
#pragma unroll
            for (int ib = 0; ib < 2; ib++) {
                const int row = wm * 64 + ib * 32 + l32;
                A[ib] = *reinterpret_cast<const half8_t *>(&xs[buf][row * kXRow + g * kGroup + 8 * half]);
            }
#pragma unroll
            for (int jb = 0; jb < 4; jb++) {
                const uint32_t pk = *reinterpret_cast<const uint32_t *>(rb + (2 * g) * (BN / 32) * 256 + jb * 256);
                const uint32_t s2 = *reinterpret_cast<const uint32_t *>(
                    rb - half * (BN / 32) * 256 + (kPkBytes / 128) * 256 + g * (BN / 32) * 256 + jb * 256);
                uint32_t bw[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t pair = lds_u32(tab, __builtin_amdgcn_perm(lanebase, pk, 0x0C0C0004u | (i << 8)));
                    bw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pair) * __builtin_bit_cast(half2_t, s2));
                }
                const half8_t B = __builtin_bit_cast(half8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
                for (int ib = 0; ib < 2; ib++)
                    acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[ib], B, acc[ib][jb], 0, 0, 0);
            }
        }
        // the other stage's readers finished before the previous step's barrier
        if (kt + 1 < nk) lstore(buf ^ 1, Rnext);
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        kstep(kt, std::integral_constant<int, 0>{}, R0, R1);
        if (kt + 1 < nk) kstep(kt + 1, std::integral_constant<int, 1>{}, R1, R0);
    }

    // ---- epilogue: lane holds column j = l32 (weight row), tokens 8(v/4) + 4 half + v%4
    const float scale = ldexpf(1.0f, ex - 8);
#pragma unroll
    for (int jb = 0; jb < 4; jb++) {
        const int64_t r = n0 + wn * 128 + jb * 32 + l32;
        if (r >= N) continue;
        const float rsc = a.s_ch[r] * scale;
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t m = m0 + wm * 64 + ib * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
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

}  // namespace

hipError_t launch_gemm_f16(const LinearArgs &a, hipStream_t stream) {
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(k_gemm_f16, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w4a8
