// Batched-decode W4A8 product for a few to 64 tokens: the weight stream of the decode GEMV
// with the multiply-accumulate on fp16 matrix cores.
//
// Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", section "Why this exists":
// decode re-reads every weight per step, so with a handful of tokens the layer is still a
// weight stream; section "Format": packed 4-bit indices into a 16-level codebook, an e4m3
// scale per 16 values, an fp32 scale per output row.
//
// Numerics (the same as the f16 prefill kernel): each weight is decoded to
// fp16(s16 * cb16[idx]) with cb16 = fp16(cb / 2^ex) (max |cb| = f 2^ex, f in [0.5, 1)) and
// s16 = s_rel * 2^8 (exact), one packed-fp16 multiply per index byte; int8 activations are
// exact in fp16; v_mfma_f32_16x16x32_f16 accumulates every group in fp32 with exact
// products, so no per-group fold is needed.  Relative error per weight <= 2^-10.
//
// Layout (gfx950):
//  * Weights are the MFMA's A side: a 16-row tile, lane (i, q) = (l % 16, l / 16) holds row
//    i.  Per 128-k half-block the lane loads 16 B of packed indices (k = 32q .. 32q+31) and
//    the two group scales of those 32 values; 4 sub-steps s take k = 32q + 8s .. +7, so the
//    MFMA's k index (8q + e) stands for k = 32q + 8s + e.
//  * Activations are the B side: lane (j, q) reads token j's x_q[k0 + 32q .. +31] (32 B,
//    L2 resident) and converts the int8 values to fp16 exactly with a byte permute and a
//    packed-fp16 subtract (bias 1152: bytes b + 128 under an fp16 exponent of 1024).
//    Tokens past M and rows past N read zero through the buffer bounds.
//  * A workgroup owns NT consecutive 16-row tiles; its waves (4 to 16, as registers allow)
//    split K (wave w takes every W-th 128-k half-block, so the waves stream adjacent pieces
//    of the same rows together) and each keeps its NT x MT16 accumulator tiles in registers.
//    Each wave's next half-block is in flight while it computes one (a ring of two; a third
//    half-block in flight was 4-11% slower at M = 8 and 32).  At the end the waves' partial
//    tiles are summed through LDS in wave order (deterministic) and scaled by
//    2^(ex-8) s_ch s_x.
//  * The codebook-pair table is the decode GEMV's (256 entries, 64 lane-private replicas).
//    Up to 48 tokens the table reads of the next row tile are issued before the current
//    tile's multiplies and MFMAs (scheduling barriers keep that order).
//  * Start-up: the codebook and the workgroup's group scales are requested before the first
//    weight loads (a request behind them waits for them to drain from HBM); the scales go
//    straight to LDS through the buffer unit (16 B per lane), so the weight stream carries
//    no 2-byte loads.
#include <type_traits>

#include <atomic>
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTiles = 5;      // 16-row tiles per workgroup
constexpr int kMaxTokTiles = 4;   // 16-token tiles (M <= 64)
constexpr int kTabBytes = 256 * 64 * 4;
constexpr int kMaxWaves = 16;
// the reduction buffer holds one token tile of every wave: WAVES x NT x 1 KiB
constexpr int kSmemBytes = kTabBytes > kMaxWaves * 4 * 1024 ? kTabBytes : kMaxWaves * 4 * 1024;
constexpr uint32_t kOutside = 0x80000000u;  // buffer offset that reads zero
constexpr int kSkinnyLdsMax = 160 * 1024;    // gfx950 LDS per workgroup
// Plain loads: each instruction reads half of every 128-B line of its 16 rows and the same
// wave reads the other half one half-block later, which must still find the line in L2.
constexpr int kNT = 0;

template <int NT, int MT16>
struct Slot {
    u32x4 pk[NT];
    u32x4 x[MT16][2];
};

// LDS bytes of a workgroup's staged group scales: whole 1 KiB blocks (one wave's copy)
__host__ __device__ __forceinline__ int64_t skinny_scale_bytes(int64_t rows, int64_t grpbytes) {
    return (rows * grpbytes + 1023) & ~(int64_t)1023;
}

__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}

// four int8 -> two fp16 pairs, exact: (b + 128) under exponent 2^10 is 1024 + b + 128
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t u = w ^ 0x80808080u;
    const half2_t bias = __builtin_bit_cast(half2_t, 0x64806480u);  // (1152, 1152)
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias);
}

template <int NT, int MT16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_skinny(LinearArgs a) {
    static_assert(WAVES * NT <= kSmemBytes / 1024, "reduction buffer");
    // pair table (later the wave reduction), then the staged group scales
    extern __shared__ __align__(16) char smem[];
    uint8_t *ss = reinterpret_cast<uint8_t *>(smem + kSmemBytes);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t r_begin = (int64_t)blockIdx.x * NT * 16;
    const int nrows = (int)min((int64_t)NT * 16, N - r_begin);
    const uint32_t rowbytes = (uint32_t)(K / 2), grpbytes = (uint32_t)(K / kGroup);

    const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.packed + r_begin * rowbytes), (short)0, (int)(nrows * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.s_rel + r_begin * grpbytes), (short)0, (int)(nrows * grpbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.x_q, (short)0, (int)(M * K), 0x00020000);

    // the codebook (four 16-byte loads of one line), then the group scales of the
    // workgroup's rows (nrows x K/16 contiguous bytes) copied to LDS 1 KiB per wave
    // instruction, all before the first weight load
    const __amdgpu_buffer_rsrc_t rs_cb = __builtin_amdgcn_make_buffer_rsrc((void *)a.cb, (short)0, kLevels * 4, 0x00020000);
    float cbv[kLevels];
#pragma unroll
    for (int q = 0; q < kLevels / 4; q++) {
        const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs_cb, 16 * q, 0, 0);
        cbv[4 * q] = __uint_as_float(c.x); cbv[4 * q + 1] = __uint_as_float(c.y);
        cbv[4 * q + 2] = __uint_as_float(c.z); cbv[4 * q + 3] = __uint_as_float(c.w);
    }
    const int nsc = (int)(nrows * grpbytes / 16);
    for (int blk = 64 * wave; blk < nsc; blk += 64 * WAVES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (__attribute__((address_space(3))) void *)(ss + 16 * blk), 16,
                                                 16u * (uint32_t)(blk + lane), 0, 0, kNT);
    __builtin_amdgcn_sched_barrier(0);

    // this wave's share of the 128-k half-blocks: every WAVES-th one, so that at any time
    // the workgroup's waves read adjacent 64-B pieces of the same rows (long DRAM runs, and
    // both halves of each 128-B line close together)
    const int nhalf = (int)(K / 128);
    const int h0 = wave, h1 = nhalf;
    constexpr int S = WAVES;

    auto fetch = [&](int h, Slot<NT, MT16> &s) {
        const bool valid = h < h1;
        const uint32_t kb = (uint32_t)h * 64u + 16u * lq;  // packed byte within the row
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const uint32_t row = (uint32_t)(16 * t + li);
            s.pk[t] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, valid ? row * rowbytes + kb : kOutside, 0, kNT);
        }
#pragma unroll
        for (int u = 0; u < MT16; u++) {
            const uint32_t off = (uint32_t)(16 * u + li) * (uint32_t)K + (uint32_t)h * 128u + 32u * lq;
            s.x[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, valid ? off : kOutside, 0, 0);
            s.x[u][1] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, valid ? off + 16u : kOutside, 0, 0);
        }
    };

    Slot<NT, MT16> R0, R1;
    fetch(h0, R0);
    fetch(h0 + S, R1);

    // codebook -> fp16 pair table scaled by 2^-ex; wave w writes 16 / WAVES high nibbles
    float cmax = 0.0f;
#pragma unroll
    for (int q = 0; q < kLevels; q++) cmax = fmaxf(cmax, fabsf(cbv[q]));
    int ex = 0;
    if (cmax > 0.0f) frexpf(cmax, &ex);
    const float inv = ldexpf(1.0f, -ex);
    uint32_t *tab = reinterpret_cast<uint32_t *>(smem);
#pragma unroll
    for (int hh = 0; hh < kLevels / WAVES; hh++) {
        const int hi_n = (kLevels / WAVES) * wave + hh;
        float cbh = 0.0f;
#pragma unroll
        for (int q = 0; q < kLevels; q++) cbh = q == hi_n ? cbv[q] : cbh;
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(cbh * inv));
#pragma unroll
        for (int lo = 0; lo < kLevels; lo++) {
            const uint32_t v = __builtin_bit_cast(uint16_t, (_Float16)(cbv[lo] * inv)) | (hi << 16);
            tab[(16 * hi_n + lo) * 64 + lane] = v;
        }
    }
    // every copy to LDS of this wave is complete once at most the two ring stages' loads
    // (issued after them) are outstanding (gfx9 s_waitcnt encoding: vmcnt in bits 3..0 and
    // 15..14, no expcnt / lgkmcnt wait); the barrier then publishes them
    constexpr int kRingLoads = 2 * (NT + 2 * MT16);
    static_assert(kRingLoads < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kRingLoads & 15) | ((kRingLoads >> 4) << 14));
    __syncthreads();

    const uint32_t lanebase = (uint32_t)lane * 4u;
    float4_t acc[NT][MT16];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int u = 0; u < MT16; u++) acc[t][u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int h, const Slot<NT, MT16> &s) {
        half8_t B[MT16][4];
#pragma unroll
        for (int u = 0; u < MT16; u++) {
            const uint32_t w[8] = {s.x[u][0].x, s.x[u][0].y, s.x[u][0].z, s.x[u][0].w,
                                   s.x[u][1].x, s.x[u][1].y, s.x[u][1].z, s.x[u][1].w};
            uint32_t f[16];
#pragma unroll
            for (int d = 0; d < 8; d++) i8x4_to_f16(w[d], f[2 * d], f[2 * d + 1]);
#pragma unroll
            for (int st = 0; st < 4; st++)
                B[u][st] = __builtin_bit_cast(half8_t, make_uint4(f[4 * st], f[4 * st + 1], f[4 * st + 2], f[4 * st + 3]));
        }
        if constexpr (MT16 <= 3) {
            // the table reads (and the scale read) of tile t + 1 go out before tile t's
            // multiplies and MFMAs, so that their LDS latency is not paid tile by tile (kept
            // off at four token tiles, where the extra registers cost more than it saves)
            uint32_t pr[2][16], srr[2];
            auto reads = [&](int t, uint32_t (&p)[16], uint32_t &sr) {
                sr = *reinterpret_cast<const uint16_t *>(ss + (16 * t + li) * grpbytes + 8u * (uint32_t)h + 2u * lq);
                const uint32_t pw[4] = {s.pk[t].x, s.pk[t].y, s.pk[t].z, s.pk[t].w};
#pragma unroll
                for (int st = 0; st < 4; st++)
#pragma unroll
                    for (int c = 0; c < 4; c++)
                        p[4 * st + c] = *reinterpret_cast<const uint32_t *>(
                            smem + __builtin_amdgcn_perm(lanebase, pw[st], 0x0C0C0004u | ((uint32_t)c << 8)));
            };
            reads(0, pr[0], srr[0]);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                if (t + 1 < NT) reads(t + 1, pr[(t + 1) & 1], srr[(t + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t sr = srr[t & 1];
                const uint32_t s0 = __builtin_bit_cast(uint16_t, (_Float16)(__builtin_amdgcn_cvt_f32_fp8((int)sr, 0) * 256.0f));
                const uint32_t s1 = __builtin_bit_cast(uint16_t, (_Float16)(__builtin_amdgcn_cvt_f32_fp8((int)sr, 1) * 256.0f));
                const uint32_t sg[2] = {s0 | (s0 << 16), s1 | (s1 << 16)};
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    uint32_t aw[4];
#pragma unroll
                    for (int c = 0; c < 4; c++) aw[c] = pk_mul(pr[t & 1][4 * st + c], sg[st >> 1]);
                    const half8_t A = __builtin_bit_cast(half8_t, make_uint4(aw[0], aw[1], aw[2], aw[3]));
#pragma unroll
                    for (int u = 0; u < MT16; u++)
                        acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[u][st], acc[t][u], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            // group scales of this lane's 32 values (row 16 t + li, groups 8 h + 2 lq and the
            // next; a row past N reads stale LDS and feeds no stored output) as fp16 pairs,
            // times 2^8 (exact for every e4m3 value)
            const uint32_t sr = *reinterpret_cast<const uint16_t *>(ss + (16 * t + li) * grpbytes + 8u * (uint32_t)h + 2u * lq);
            const uint32_t s0 = __builtin_bit_cast(uint16_t, (_Float16)(__builtin_amdgcn_cvt_f32_fp8((int)sr, 0) * 256.0f));
            const uint32_t s1 = __builtin_bit_cast(uint16_t, (_Float16)(__builtin_amdgcn_cvt_f32_fp8((int)sr, 1) * 256.0f));
            const uint32_t sg[2] = {s0 | (s0 << 16), s1 | (s1 << 16)};
            const uint32_t pw[4] = {s.pk[t].x, s.pk[t].y, s.pk[t].z, s.pk[t].w};
#pragma unroll
            for (int st = 0; st < 4; st++) {
                uint32_t aw[4];
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const uint32_t pair = *reinterpret_cast<const uint32_t *>(
                        smem + __builtin_amdgcn_perm(lanebase, pw[st], 0x0C0C0004u | ((uint32_t)c << 8)));
                    aw[c] = pk_mul(pair, sg[st >> 1]);
                }
                const half8_t A = __builtin_bit_cast(half8_t, make_uint4(aw[0], aw[1], aw[2], aw[3]));
#pragma unroll
                for (int u = 0; u < MT16; u++)
                    acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[u][st], acc[t][u], 0, 0, 0);
            }
        }
        }
    };

    // Fetches are unconditional (half-blocks past the range read zero) so the number of
    // loads in flight is the same on every path and each compute waits only for its own.
    for (int h = h0; h < h1; h += 2 * S) {
        compute(h, R0);
        fetch(h + 2 * S, R0);
        if (h + S < h1) compute(h + S, R1);
        fetch(h + 3 * S, R1);
    }
    // Wave partials are summed through LDS one token tile at a time, in wave order
    // (deterministic): [wave][t][lane] float4, lane holding rows 4 lq .. 4 lq + 3 of the
    // tile for token li.  Threads 0..255 then own (token j, row i) of each tile, rows
    // fastest, so consecutive threads store consecutive y elements.
    float4_t *red = reinterpret_cast<float4_t *>(smem);
    const float scale = ldexpf(1.0f, ex - 8);
    const int i = tid & 15, j = (tid >> 4) & 15;
    const int src = 16 * (i >> 2) + j, comp = i & 3;
    float rsc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int64_t r = r_begin + 16 * t + i;
        rsc[t] = r < N ? a.s_ch[r] * scale : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < MT16; u++) {
        __syncthreads();  // the table, or the previous token tile, is no longer read
#pragma unroll
        for (int t = 0; t < NT; t++) red[(wave * NT + t) * 64 + lane] = acc[t][u];
        __syncthreads();
        const int64_t m = 16 * u + j;
        if (tid < 256 && m < M) {
            const float sxm = a.s_x[m];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const int64_t r = r_begin + 16 * t + i;
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES; w++) v += red[(w * NT + t) * 64 + src][comp];
                if (r < N) {
                    const float val = (v * rsc[t]) * sxm;
                    if (a.y_bf16)
                        static_cast<uint16_t *>(a.y)[m * N + r] = f32_to_bf16_rne(val);
                    else
                        static_cast<float *>(a.y)[m * N + r] = val;
                }
            }
        }
    }
}

// Waves per workgroup: as many as the registers allow (each wave takes a share of K), so
// that every SIMD has several waves to hide LDS and matrix-core latency.
template <int NT, int MT16>
constexpr int waves_for() { return (MT16 == 1 && NT <= 3) ? 16 : (MT16 <= 2 ? 8 : 4); }

template <int NT, int MT16>
hipError_t launch_one(const LinearArgs &a, unsigned grid, hipStream_t stream) {
    constexpr int W = waves_for<NT, MT16>();
    const int64_t lds = kSmemBytes + skinny_scale_bytes(16 * NT, a.K / kGroup);
    // set once per kernel instance; concurrent first calls may both set it, which is harmless
    static std::atomic<bool> attr_set{false};
    if (!attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_skinny<NT, MT16, W>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kSkinnyLdsMax);
        if (e != hipSuccess) return e;
        attr_set.store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((k_skinny<NT, MT16, W>), dim3(grid), dim3(64 * W), (size_t)lds, stream, a);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(const LinearArgs &a, unsigned grid, hipStream_t stream) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_one<NT, 1>(a, grid, stream);
        case 2: return launch_one<NT, 2>(a, grid, stream);
        case 3: return launch_one<NT, 3>(a, grid, stream);
        case 4: return launch_one<NT, 4>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool skinny_supported(int64_t M, int64_t N, int64_t K) {
    // 32-bit buffer offsets: token rows of x_q and a workgroup's rows of packed data; LDS:
    // the table plus the staged group scales of kMaxTiles row tiles
    return M >= 1 && M <= 16 * kMaxTokTiles && M * K < (int64_t(1) << 31) &&
           (int64_t)16 * kMaxTiles * (K / 2) < (int64_t(1) << 31) && N >= 1 &&
           kSmemBytes + skinny_scale_bytes(16, K / kGroup) <= kSkinnyLdsMax;
}

hipError_t launch_gemm_skinny(const LinearArgs &a, int num_cu, hipStream_t stream) {
    if (!skinny_supported(a.M, a.N, a.K)) return hipErrorInvalidValue;
    // tiles per workgroup: enough to give every CU one workgroup, at most kMaxTiles
    const int64_t tiles = (a.N + 15) / 16;
    // (fewer for long rows: the staged scales of a workgroup's rows must fit in LDS)
    int64_t nt = (tiles + num_cu - 1) / num_cu;
    if (nt > kMaxTiles) nt = kMaxTiles;
    while (nt > 1 && kSmemBytes + skinny_scale_bytes(16 * nt, a.K / kGroup) > kSkinnyLdsMax) nt--;
    if (nt < 1) nt = 1;
    const unsigned grid = (unsigned)((tiles + nt - 1) / nt);
    switch (nt) {
        case 1: return launch_nt<1>(a, grid, stream);
        case 2: return launch_nt<2>(a, grid, stream);
        case 3: return launch_nt<3>(a, grid, stream);
        case 4: return launch_nt<4>(a, grid, stream);
        default: return launch_nt<5>(a, grid, stream);
    }
}

}  // namespace w4a8
