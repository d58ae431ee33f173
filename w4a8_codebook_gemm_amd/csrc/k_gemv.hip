// Kernel 2: decode GEMV for small token counts (M <= 4) -- streams the packed 4-bit
// weights once from HBM and fuses nibble unpack, codebook lookup, the per-16 fp8 group
// scale and the per-row scale.
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", section "Why this exists":
// generation is bandwidth bound because every token re-reads all weights; the layer adds
// a codebook dequantisation step on top of the int8 product (section "Format": packed
// indices into a 16-level fp32 codebook, an e4m3 scale per 16 values, an fp32 scale per
// output row).
//
// Design (gfx950):
//  * Persistent grid: one 1024-thread workgroup per CU owns a contiguous range of rows,
//    so each CU streams one contiguous stretch of the packed matrix.
//  * The unit of work is (row pair, 256-wide K block): 8 lanes each load 16 B (32 indices,
//    two groups) of both rows -- every load instruction covers whole 128-B lines.
//  * Codebook lookup: an LDS table of 256 entries, one per possible packed byte, holding
//    the fp16 pair (cb[low nibble], cb[high nibble]) scaled by a power of two so the
//    largest level lies in [0.5, 1).  The table is replicated 64 times so that lane c
//    always reads bank c: the index byte goes to address bits 8..15 and the lane id to
//    bits 2..7 in one v_perm, the read is conflict-free, and one v_dot2_f32_f16 with the
//    fp16 pair of activations (int8 values, exact in fp16) gives two products with fp32
//    accumulation.  Relative error of the fp16 codebook is at most 2^-11 per level.
//  * Each group's two-element dot products are summed in fp32, scaled by the decoded e4m3
//    group scale, reduced over the 8 lanes with xor shuffles, and written to an LDS
//    partial per (row, block); one thread per row then sums its partials in block order
//    and applies s_channel, s_x and the codebook's power-of-two scale.  No atomics: the
//    result is deterministic.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 1024;
constexpr int kLaneGroups = kThreads / 8;
constexpr int kTabWords = 256 * 64;                 // 64 KiB
constexpr int kLdsMax = 160 * 1024;                 // gfx950 LDS per workgroup
constexpr int kMaxMT = 4;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

__device__ __forceinline__ uint32_t tab_read(const uint32_t *lds, uint32_t byte_addr) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lds) + byte_addr);
}

// 16 packed bytes of one row against MT token vectors: two groups of 16 products each.
template <int MT>
__device__ __forceinline__ void row_block(const uint32_t *lds, uint32_t lanebase, const uint4 &p,
                                          const uint32_t (&xv)[MT][16], float (&g0)[MT],
                                          float (&g1)[MT]) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int m = 0; m < MT; m++) g0[m] = g1[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t addr = __builtin_amdgcn_perm(lanebase, w[i >> 2], 0x0C0C0004u | ((i & 3) << 8));
        const uint32_t pair = tab_read(lds, addr);
#pragma unroll
        for (int m = 0; m < MT; m++) {
            if (i < 8) g0[m] = dot2(pair, xv[m][i], g0[m]);
            else g1[m] = dot2(pair, xv[m][i], g1[m]);
        }
    }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void k_gemv(LinearArgs a, int rows_per_wg) {
    extern __shared__ uint32_t lds[];
    const int tid = threadIdx.x;
    const int64_t K = a.K, N = a.N;
    const int nblk = (int)(K / kRot);
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrow = (int)min((int64_t)rows_per_wg, N - r0);
    uint32_t *xs = lds + kTabWords;                              // [MT][K/2] fp16 pairs
    float *part = reinterpret_cast<float *>(xs + MT * (K / 2));  // [MT][rows_per_wg][nblk]

    // codebook -> fp16 pair table, scaled by 2^-ex with max |cb| = f * 2^ex, f in [0.5, 1)
    float cmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kLevels; j++) cmax = fmaxf(cmax, fabsf(a.cb[j]));
    int ex = 0;
    if (cmax > 0.0f) frexpf(cmax, &ex);
    const float inv = ldexpf(1.0f, -ex);
    uint32_t h[kLevels];
#pragma unroll
    for (int j = 0; j < kLevels; j++)
        h[j] = __builtin_bit_cast(uint16_t, (_Float16)(a.cb[j] * inv));
    for (int i = tid; i < kTabWords; i += kThreads) {
        const int e = i >> 6;
        lds[i] = h[e & 15] | (h[e >> 4] << 16);
    }
    // activations int8 -> fp16 pairs (exact)
    const uint32_t *xq4 = reinterpret_cast<const uint32_t *>(a.x_q);
    for (int64_t i = tid; i < MT * (K / 4); i += kThreads) {
        const uint32_t w = xq4[i];
        uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(int8_t)(w & 0xFF)) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int8_t)((w >> 8) & 0xFF)) << 16);
        uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(int8_t)((w >> 16) & 0xFF)) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int8_t)(w >> 24)) << 16);
        xs[2 * i] = lo;
        xs[2 * i + 1] = hi;
    }
    __syncthreads();

    const int lg = tid >> 3, j = tid & 7;
    const uint32_t lanebase = (uint32_t)(tid & 63) * 4u;
    const int npairs = (nrow + 1) >> 1;
    const int units = npairs * nblk;
    const int64_t rowbytes = K / 2, grpbytes = K / kGroup;
    for (int u = lg; u < units; u += kLaneGroups) {
        const int rp = u / nblk, t = u - rp * nblk;
        const int rla = 2 * rp, rlb = rla + 1;
        const bool hasb = rlb < nrow;
        const int64_t ra = r0 + rla, rb = hasb ? ra + 1 : ra;
        const int64_t koff = (int64_t)t * 128 + 16 * j;
        const uint4 pa = *reinterpret_cast<const uint4 *>(a.packed + ra * rowbytes + koff);
        const uint4 pb = *reinterpret_cast<const uint4 *>(a.packed + rb * rowbytes + koff);
        const uint32_t sa = *reinterpret_cast<const uint16_t *>(a.s_rel + ra * grpbytes + t * 16 + 2 * j);
        const uint32_t sb = *reinterpret_cast<const uint16_t *>(a.s_rel + rb * grpbytes + t * 16 + 2 * j);
        uint32_t xv[MT][16];
#pragma unroll
        for (int m = 0; m < MT; m++) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xs + m * (K / 2) + koff);
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const uint4 v = src[c];
                xv[m][4 * c + 0] = v.x; xv[m][4 * c + 1] = v.y;
                xv[m][4 * c + 2] = v.z; xv[m][4 * c + 3] = v.w;
            }
        }
        float ga0[MT], ga1[MT], gb0[MT], gb1[MT];
        row_block<MT>(lds, lanebase, pa, xv, ga0, ga1);
        row_block<MT>(lds, lanebase, pb, xv, gb0, gb1);
        const float sa0 = e4m3_to_f32(sa & 0xFF), sa1 = e4m3_to_f32(sa >> 8);
        const float sb0 = e4m3_to_f32(sb & 0xFF), sb1 = e4m3_to_f32(sb >> 8);
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float va = sa0 * ga0[m] + sa1 * ga1[m];
            float vb = sb0 * gb0[m] + sb1 * gb1[m];
#pragma unroll
            for (int s = 1; s < 8; s <<= 1) {
                va += __shfl_xor(va, s);
                vb += __shfl_xor(vb, s);
            }
            if (j == 0) {
                part[(m * rows_per_wg + rla) * nblk + t] = va;
                if (hasb) part[(m * rows_per_wg + rlb) * nblk + t] = vb;
            }
        }
    }
    __syncthreads();

    const float cbscale = ldexpf(1.0f, ex);
    for (int i = tid; i < MT * nrow; i += kThreads) {
        const int m = i / nrow, rl = i - m * nrow;
        const float *pp = part + (m * rows_per_wg + rl) * nblk;
        float acc = 0.0f;
        for (int t = 0; t < nblk; t++) acc += pp[t];
        const int64_t r = r0 + rl;
        const float v = ((acc * a.s_ch[r]) * a.s_x[m]) * cbscale;
        if (a.y_bf16)
            static_cast<uint16_t *>(a.y)[m * N + r] = f32_to_bf16_rne(v);
        else
            static_cast<float *>(a.y)[m * N + r] = v;
    }
}

template <int MT>
hipError_t launch_mt(const LinearArgs &a, int num_cu, hipStream_t stream) {
    const int64_t nblk = a.K / kRot;
    const int64_t fixed = (int64_t)kTabWords * 4 + (int64_t)MT * a.K * 2;
    int64_t rows = (a.N + num_cu - 1) / num_cu;
    rows += rows & 1;
    while (rows > 2 && fixed + (int64_t)MT * rows * nblk * 4 > kLdsMax) rows = ((rows / 2) + 1) & ~1LL;
    const int64_t lds = fixed + (int64_t)MT * rows * nblk * 4;
    if (lds > kLdsMax) return hipErrorInvalidValue;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemv<MT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const unsigned grid = (unsigned)((a.N + rows - 1) / rows);
    hipLaunchKernelGGL(k_gemv<MT>, dim3(grid), dim3(kThreads), (size_t)lds, stream, a, (int)rows);
    return hipGetLastError();
}

}  // namespace

bool gemv_supported(int64_t M, int64_t K) { return M >= 1 && M <= kMaxMT && M * K <= 40960; }

hipError_t launch_gemv(const LinearArgs &a, int num_cu, hipStream_t stream) {
    switch (a.M) {
        case 1: return launch_mt<1>(a, num_cu, stream);
        case 2: return launch_mt<2>(a, num_cu, stream);
        case 3: return launch_mt<3>(a, num_cu, stream);
        case 4: return launch_mt<4>(a, num_cu, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a8
