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
// s16 = s_rel * 2^7 (exact, below 65504 for every finite e4m3 value), one packed-fp16
// multiply per index byte; int8 activations are
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
//  * One workgroup per compute unit: each owns ceil(N / CUs) consecutive rows as NT 16-row
//    tiles, the last one partial (its rows past the workgroup's range read zero through the
//    buffer bounds and are never stored), so every CU streams an equal share; its waves (4 to
//    16, as registers allow)
//    split K (wave w takes every W-th 128-k half-block, so the waves stream adjacent pieces
//    of the same rows together) and each keeps its NT x MT16 accumulator tiles in registers.
//    Each wave's next half-block is in flight while it computes one (a ring of two; a third
//    half-block in flight was 4-11% slower at M = 8 and 32).  At the end the waves' partial
//    tiles are summed through LDS in wave order (deterministic) and scaled by
//    2^(ex-7) s_ch s_x.
//  * The codebook-pair table is the decode GEMV's (256 entries, 64 lane-private replicas).
//    Up to 48 tokens the table reads of the next row tile are issued before the current
//    tile's multiplies and MFMAs (scheduling barriers keep that order).
//  * K split (w4a8_linear_ws, with a caller's workspace): where a CU would own few rows, K is
//    cut into parts and each workgroup takes full row tiles over one part.  Each part
//    stores its unscaled sums with device-scope relaxed atomic stores (written through to
//    the point where every XCD sees them, without a cache-wide flush), then counts its
//    arrival on the row block's counter; the last part to arrive reads every part's sums,
//    adds them in part order and writes y, and the counter wraps back to zero.
//  * Start-up: the epilogue's row and token scales, then the workgroup's group scales are
//    requested before the first weight loads (a request behind them waits for them to drain
//    from HBM); the group scales go straight to LDS through the buffer unit (16 B per lane),
//    so the weight stream carries no 2-byte loads.  The codebook comes through the scalar
//    cache, outside the in-order vector load counter.  The pair table sits in static LDS, so
//    its address is a constant of every table read.
#include <type_traits>

#include <atomic>
#include "e4m3_pair.h"
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

// Layers of one launch (all with the same N): layer g owns workgroups [g nrb, (g + 1) nrb),
// each running exactly what the single-layer launch runs for its row block.
struct SkinnyTab {
    int G, nrb;
    LayerDesc L[kMaxGroup];
};

template <int NT, int MT16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_skinny(LinearArgs a, int rows_wg, SkinnyTab lt) {
    static_assert(WAVES * NT <= kSmemBytes / 1024, "reduction buffer");
    // pair table (later the wave reduction) in static LDS, whose address folds into every
    // table read; the staged group scales in the dynamic part
    __shared__ __align__(16) uint32_t tabs[kSmemBytes / 4];
    extern __shared__ __align__(16) char dyn[];
    char *smem = reinterpret_cast<char *>(tabs);
    uint8_t *ss = reinterpret_cast<uint8_t *>(dyn);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int64_t M = a.M, N = a.N, K = a.K;
    // with a split of K, workgroup b takes part ks = b % ksplit of K for row block b / ksplit
    int bid = (int)blockIdx.x;
    if (lt.G > 1) {
        // this workgroup's layer (compile-time indices keep the table in kernel arguments)
        const int g = bid / lt.nrb;
        bid -= g * lt.nrb;
#pragma unroll
        for (int q = 0; q < kMaxGroup; q++)
            if (q == g) {
                a.packed = lt.L[q].packed;
                a.s_rel = lt.L[q].s_rel;
                a.s_ch = lt.L[q].s_ch;
                a.cb = lt.L[q].cb;
                a.y = lt.L[q].y;
            }
    }
    const int ksplit = a.ksplit > 1 ? a.ksplit : 1;
    const int ks = bid % ksplit, rb = bid / ksplit;
    const int64_t r_begin = (int64_t)rb * rows_wg;
    const int nrows = (int)min((int64_t)rows_wg, N - r_begin);
    const uint32_t rowbytes = (uint32_t)(K / 2), grpbytes = (uint32_t)(K / kGroup);
    const uint32_t grs = grpbytes / (uint32_t)ksplit;  // group-scale bytes of a row in this part

    const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.packed + r_begin * rowbytes), (short)0, (int)(nrows * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.s_rel + r_begin * grpbytes), (short)0, (int)(nrows * grpbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.x_q, (short)0, (int)(M * K), 0x00020000);

    // the epilogue's row and token scales, requested before anything else: thread (i, j) of
    // the final sums owns row 16 t + i and token 16 u + j (rows past the range, tokens past
    // M and threads past 256 read zero through the buffer bounds)
    const int ei = tid & 15, ej = (tid >> 4) & 15;
    float rsc[NT], sxv[MT16];
    {
        const __amdgpu_buffer_rsrc_t rs_c = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.s_ch + r_begin), (short)0, (int)(nrows * 4), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs_sx = __builtin_amdgcn_make_buffer_rsrc((void *)a.s_x, (short)0, (int)(M * 4), 0x00020000);
#pragma unroll
        for (int t = 0; t < NT; t++)
            rsc[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_c, (uint32_t)(16 * t + ei) * 4u, 0, 0));
#pragma unroll
        for (int u = 0; u < MT16; u++)
            sxv[u] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rs_sx, tid < 256 ? (uint32_t)(16 * u + ej) * 4u : kOutside, 0, 0));
    }

    // the codebook (scalar loads), then the group scales of the workgroup's rows (nrows x
    // K/16 contiguous bytes) copied to LDS 1 KiB per wave instruction, all before the first
    // weight load
    const __attribute__((address_space(4))) float *cbk = (const __attribute__((address_space(4))) float *)a.cb;
    float cbv[kLevels];
#pragma unroll
    for (int q = 0; q < kLevels; q++) cbv[q] = cbk[q];
    const int nsc = (int)(nrows * grs / 16);
    const uint32_t cpr = grs / 16;  // 16-byte chunks per row of this part
    for (int blk = 64 * wave; blk < nsc; blk += 64 * WAVES) {
        const uint32_t c = (uint32_t)(blk + lane), row = c / cpr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (__attribute__((address_space(3))) void *)(ss + 16 * blk), 16,
                                                 row * grpbytes + (uint32_t)ks * grs + 16u * (c - row * cpr), 0, 0, kNT);
    }
    __builtin_amdgcn_sched_barrier(0);

    // this wave's share of the 128-k half-blocks: every WAVES-th one, so that at any time
    // the workgroup's waves read adjacent 64-B pieces of the same rows (long DRAM runs, and
    // both halves of each 128-B line close together)
    const int nhalf = (int)(K / 128) / ksplit, hb = ks * nhalf;  // this part's half-blocks
    const int h0 = wave, h1 = nhalf;
    constexpr int S = WAVES;

    auto fetch = [&](int h, Slot<NT, MT16> &s) {
        const bool valid = h < h1;
        const uint32_t kb = (uint32_t)(hb + h) * 64u + 16u * lq;  // packed byte within the row
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const uint32_t row = (uint32_t)(16 * t + li);
            s.pk[t] = __builtin_amdgcn_raw_buffer_load_b128(rs_p, valid ? row * rowbytes + kb : kOutside, 0, kNT);
        }
#pragma unroll
        for (int u = 0; u < MT16; u++) {
            const uint32_t off = (uint32_t)(16 * u + li) * (uint32_t)K + (uint32_t)(hb + h) * 128u + 32u * lq;
            s.x[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, valid ? off : kOutside, 0, 0);
            s.x[u][1] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, valid ? off + 16u : kOutside, 0, 0);
        }
    };

    // every wave's first slot goes out before any wave's second, so that the first
    // half-blocks of all waves arrive first and the waves start together (a bare barrier
    // orders the issue only)
    Slot<NT, MT16> R0, R1;
    fetch(h0, R0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
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
                sr = *reinterpret_cast<const uint16_t *>(ss + (16 * t + li) * grs + 8u * (uint32_t)h + 2u * lq);
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
                const uint32_t s2 = e4m3x2_to_f16x2(srr[t & 1], 128.0f);
                const uint32_t sg[2] = {__builtin_amdgcn_perm(0u, s2, 0x01000100u), __builtin_amdgcn_perm(0u, s2, 0x03020302u)};
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
            // times 2^7 (exact for every e4m3 value, and at most 448 * 2^7 = 57344)
            const uint32_t sr = *reinterpret_cast<const uint16_t *>(ss + (16 * t + li) * grs + 8u * (uint32_t)h + 2u * lq);
            const uint32_t s2 = e4m3x2_to_f16x2(sr, 128.0f);
            const uint32_t sg[2] = {__builtin_amdgcn_perm(0u, s2, 0x01000100u), __builtin_amdgcn_perm(0u, s2, 0x03020302u)};
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
    const float scale = ldexpf(1.0f, ex - 7);
    const int src = 16 * (ei >> 2) + ej, comp = ei & 3;
#pragma unroll
    for (int t = 0; t < NT; t++) rsc[t] *= scale;
#pragma unroll
    for (int u = 0; u < MT16; u++) {
        __syncthreads();  // the table, or the previous token tile, is no longer read
#pragma unroll
        for (int t = 0; t < NT; t++) red[(wave * NT + t) * 64 + lane] = acc[t][u];
        __syncthreads();
        const int64_t m = 16 * u + ej;
        if (tid < 256 && m < M) {
            const float sxm = sxv[u];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const int64_t r = r_begin + 16 * t + ei;
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES; w++) v += red[(w * NT + t) * 64 + src][comp];
                if (r < r_begin + nrows) {
                    if (ksplit > 1) {
                        // this part's sum, stored coherently across XCDs (device-scope atomic
                        // store: written through the XCD's L2, no cache-wide flush)
                        __hip_atomic_store(a.ws_part + ((int64_t)ks * M + m) * N + r, v, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    } else {
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
    if (ksplit > 1) {
        // The last part of the row block to arrive adds the parts' sums in part order (so
        // the result does not depend on the order of arrival) and writes y.  The counter
        // wraps to 0 on the last arrival, leaving the workspace as it was found.
        // the flag lives in the staged-scale area (no longer read): a static LDS variable
        // would push static + dynamic LDS past the 160 KiB the launch asks for
        int *last = reinterpret_cast<int *>(dyn);
        // every store of this part has completed (reached the device's coherence point)
        // before its arrival counts; the loads of the last part are issued after the count
        // that makes it last, so they see every part.  Device-scope fences would instead
        // write back and invalidate the whole L2 of every XCD.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) *last = atomicInc(a.ws_cnt + rb, (unsigned)(ksplit - 1)) == (unsigned)(ksplit - 1);
        __syncthreads();
        if (*last) {
            // every part's sums of all this thread's outputs are requested at once (one
            // memory round trip), then added in part order
            constexpr int kMaxParts = 4;
            float pv[MT16][NT][kMaxParts];
#pragma unroll
            for (int u = 0; u < MT16; u++)
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const int64_t m = 16 * u + ej, r = r_begin + 16 * t + ei;
                    const bool ok = tid < 256 && m < M && r < r_begin + nrows;
#pragma unroll
                    for (int q = 0; q < kMaxParts; q++)
                        pv[u][t][q] = ok && q < ksplit ? __hip_atomic_load(a.ws_part + ((int64_t)q * M + m) * N + r,
                                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                       : 0.0f;
                }
#pragma unroll
            for (int u = 0; u < MT16; u++)
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const int64_t m = 16 * u + ej, r = r_begin + 16 * t + ei;
                    if (tid < 256 && m < M && r < r_begin + nrows) {
                        float v = pv[u][t][0];
#pragma unroll
                        for (int q = 1; q < kMaxParts; q++)
                            if (q < ksplit) v += pv[u][t][q];
                        const float val = (v * rsc[t]) * sxv[u];
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
hipError_t launch_one(const LinearArgs &a, unsigned grid, int rows_wg, const SkinnyTab &tab, hipStream_t stream) {
    constexpr int W = waves_for<NT, MT16>();
    const int64_t lds = skinny_scale_bytes(rows_wg, a.K / kGroup / (a.ksplit > 1 ? a.ksplit : 1));
    // set once per kernel instance; concurrent first calls may both set it, which is harmless
    static std::atomic<bool> attr_set{false};
    if (!attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_skinny<NT, MT16, W>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kSkinnyLdsMax - kSmemBytes);
        if (e != hipSuccess) return e;
        attr_set.store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((k_skinny<NT, MT16, W>), dim3(grid), dim3(64 * W), (size_t)lds, stream, a, rows_wg, tab);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(const LinearArgs &a, unsigned grid, int rows_wg, const SkinnyTab &tab, hipStream_t stream) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_one<NT, 1>(a, grid, rows_wg, tab, stream);
        case 2: return launch_one<NT, 2>(a, grid, rows_wg, tab, stream);
        case 3: return launch_one<NT, 3>(a, grid, rows_wg, tab, stream);
        case 4: return launch_one<NT, 4>(a, grid, rows_wg, tab, stream);
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

int skinny_split(int64_t M, int64_t N, int64_t K, int num_cu) {
    // K split into 4 parts when a workgroup would otherwise own few rows and K is long: each
    // part then takes up to kMaxTiles full tiles over a quarter of K, so every CU reads a
    // quarter of the activations and no tile is mostly padding; each wave keeps at least two
    // half-blocks of its part.  Measured on the sweep shapes, the split pays from 17 tokens
    // on (5120 x 17408); with two parts, or fewer tokens, the parts' final sums cost more
    // than it saves.
    constexpr int q = 4;
    if (!skinny_supported(M, N, K) || M <= 16) return 1;
    const int64_t rows1 = (N + num_cu - 1) / num_cu, rows = (N * q + num_cu - 1) / num_cu;
    if (rows <= 16 * kMaxTiles && rows > rows1 && K % (256 * q) == 0 && K / 128 / q >= 16 &&
        kSmemBytes + skinny_scale_bytes(rows, K / kGroup / q) <= kSkinnyLdsMax &&
        (N + rows - 1) / rows <= kSkinnyCounterBytes / 4)
        return q;
    return 1;
}

int64_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int num_cu) {
    // the arrival counters first, at a fixed place and size whatever the shape (so that a
    // workspace can serve shapes of different sizes: no part's sums ever land on a counter),
    // then the parts' sums
    const int q = skinny_split(M, N, K, num_cu);
    return q == 1 ? 0 : kSkinnyCounterBytes + (int64_t)q * M * N * 4;
}

namespace {

// One launch of G layers of N rows each (G = 1: the layer in a).
hipError_t launch_skinny_layers(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu, hipStream_t stream) {
    if (!skinny_supported(a.M, a.N, a.K) || G < 1 || G > kMaxGroup) return hipErrorInvalidValue;
    if (G > 1 && a.ksplit > 1) return hipErrorInvalidValue;
    const int q = a.ksplit > 1 ? a.ksplit : 1;
    if (q > 1 && (a.K % (256 * q) != 0 || !a.ws_part || !a.ws_cnt)) return hipErrorInvalidValue;
    // rows per workgroup: an equal share for every CU (per part of K), at most kMaxTiles
    // tiles
    int64_t rows = (a.N * q + num_cu - 1) / num_cu;
    if (rows > 16 * kMaxTiles) rows = 16 * kMaxTiles;
    while (rows > 16 && kSmemBytes + skinny_scale_bytes(rows, a.K / kGroup / q) > kSkinnyLdsMax) rows -= 16;
    if (rows < 1) rows = 1;
    const int64_t nt = (rows + 15) / 16;
    const int64_t nrb = ((a.N + rows - 1) / rows) * q;   // workgroups per layer
    SkinnyTab tab{};
    tab.G = G;
    tab.nrb = (int)nrb;
    for (int g = 0; g < G && layers; g++) tab.L[g] = layers[g];
    const unsigned grid = (unsigned)(nrb * G);
    switch (nt) {
        case 1: return launch_nt<1>(a, grid, (int)rows, tab, stream);
        case 2: return launch_nt<2>(a, grid, (int)rows, tab, stream);
        case 3: return launch_nt<3>(a, grid, (int)rows, tab, stream);
        case 4: return launch_nt<4>(a, grid, (int)rows, tab, stream);
        default: return launch_nt<5>(a, grid, (int)rows, tab, stream);
    }
}

}  // namespace

hipError_t launch_gemm_skinny(const LinearArgs &a, int num_cu, hipStream_t stream) {
    return launch_skinny_layers(a, nullptr, 1, num_cu, stream);
}

hipError_t launch_gemm_skinny_multi(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu,
                                    hipStream_t stream) {
    for (int g = 0; g < G; g++)
        if (layers[g].N != a.N) return hipErrorInvalidValue;
    return launch_skinny_layers(a, layers, G, num_cu, stream);
}

}  // namespace w4a8
