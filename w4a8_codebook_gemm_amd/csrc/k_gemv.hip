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
//  * Latency: each 8-lane group issues two units (512 B) before the prologue, so their
//    HBM latency overlaps the table build; from then on one unit is in flight while one is
//    computed (its loads go out before the compute).  More bytes in flight than that only
//    adds contention in HBM.  The weight stream uses non-temporal buffer loads with
//    workgroup-relative 32-bit offsets.
//  * Units run in row-major order, so a wave reads 1 KiB contiguous per row; the group
//    scales of the workgroup's rows are copied to LDS up front by the buffer unit (16 B per
//    lane); the activation chunks in LDS are XOR-swizzled by lane and by block parity so
//    that the two groups served together cover all 64 LDS banks.
//  * Each group's two-element dot products are summed in fp32, scaled by the decoded e4m3
//    group scale, reduced over the 8 lanes with xor shuffles, and written to an LDS
//    partial per (row, block) (odd row stride: conflict-free); eight lanes per row then
//    sum its partials in a fixed order and apply s_channel (loaded at kernel start), s_x
//    and the codebook's power-of-two scale.  No atomics: the result is deterministic.
//  * Start-up: every small operand (row scales, activations, group scales) is requested
//    before the first weight loads; a request issued behind them would wait in the in-order
//    vector load counter for the first weight traffic to drain from HBM before the prologue
//    could use it.  The codebook is read with scalar loads, outside that counter.
#include <atomic>
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 1024;
constexpr int kLaneGroups = kThreads / 8;
constexpr int kTabWords = 256 * 64;                 // 64 KiB
constexpr int kLdsMax = 160 * 1024;                 // gfx950 LDS per workgroup
constexpr int kMaxMT = 4;
constexpr int kMaxXChunks = 40960 / 8 / kThreads;  // 8-value activation chunks per thread
constexpr int kScaleLoads = 4;                     // 16-byte group-scale loads per thread: <= 64 KiB per workgroup
// Activation words per 256-wide K block in LDS (128 fp16 pairs, unpadded).  Lane j of a
// group reads the 16 words 16j .. 16j+15 of its block as four 4-word chunks, chunk c stored
// at position c ^ ((j >> 1) & 3) ^ (block & 1): the 8 lanes of one group cover 32 of the 64
// banks and the group on the next block (the other 8 lanes served in the same cycle of a
// 16-byte read) the other 32.
constexpr int kXBlk = 128;

__device__ __forceinline__ int xchunk_swizzle(int j, int block) { return ((j >> 1) & 3) ^ (block & 1); }
// Fused activation preparation keeps a token's rotated row in registers: 64 lane rows of
// 16 x 2 rounds of 256-blocks, so K <= 32768.
constexpr int kFusedRounds = 2;

template <int MT>
constexpr int depth() { return 2; }

// LDS bytes of the staged group scales: whole 1 KiB blocks (one wave's copy)
__host__ __device__ __forceinline__ int64_t scale_lds_bytes(int64_t rows, int64_t grpbytes) {
    return (rows * grpbytes + 1023) & ~(int64_t)1023;
}  // units in flight per 8-lane group (more only adds contention)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

__device__ __forceinline__ uint32_t tab_read(const uint32_t *lds, uint32_t byte_addr) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lds) + byte_addr);
}

// The fp16 codebook pairs of both rows of a unit (2 x 16 packed bytes): all 32 table reads
// are issued together so one LDS round trip covers the whole unit.
__device__ __forceinline__ void unit_pairs(const uint32_t *lds, uint32_t lanebase, const u32x4 &pa,
                                           const u32x4 &pb, uint32_t (&pair)[32]) {
    const uint32_t w[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
    for (int i = 0; i < 32; i++)
        pair[i] = tab_read(lds, __builtin_amdgcn_perm(lanebase, w[i >> 2], 0x0C0C0004u | ((i & 3) << 8)));
}

// One token's group partials g[row][group] of a unit; each group's 8 products are split over
// two accumulators to shorten the dependency chain.
__device__ __forceinline__ void unit_dots(const uint32_t (&pair)[32], const uint32_t (&xv)[16], float (&g)[2][2]) {
#pragma unroll
    for (int r = 0; r < 2; r++) {
#pragma unroll
        for (int gi = 0; gi < 2; gi++) {
            float e0 = 0.0f, e1 = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; q += 2) {
                e0 = dot2(pair[16 * r + 8 * gi + q], xv[8 * gi + q], e0);
                e1 = dot2(pair[16 * r + 8 * gi + q + 1], xv[8 * gi + q + 1], e1);
            }
            g[r][gi] = e0 + e1;
        }
    }
}

// 8-lane sum with DPP adds (no LDS traffic): lanes of a quad exchange over distances 1 and
// 2, then lane 8k adds the quad of lane 8k+4 (row rotate by 12).  Lane 8k ends with the
// sum of lanes 8k..8k+7.
__device__ __forceinline__ float sum8_to_leader(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x12C, 0xF, 0xF, false));  // row_ror:12
    return v;
}

// Maximum over the 64 lanes of a wave of non-negative values (exact in any order): DPP
// within each 16-lane row, then the four row maxima read as scalars.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));  // row_ror:4
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));  // row_ror:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The int8 activations of sixteen rotated values as clamped integers in fp32, with the
// arithmetic of quant16_auto (bit-identical results): the exactly corrected reciprocal
// when s >= kQuantFastMin, IEEE division otherwise, all zero when the token is zero.
__device__ __forceinline__ void quant16_values(const float v[16], float s, float r, bool nonzero, float q[16]) {
    const bool fast = s >= kQuantFastMin;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        float t;
        if (fast) {
            const float q0 = v[i] * r;
            const float e = fmaf(-q0, s, v[i]);
            t = rintf(fmaf(e, r, q0));
        } else {
            t = rintf(v[i] / s);
        }
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        q[i] = nonzero ? t : 0.0f;
    }
}

// One ring slot: buffer offsets of a unit for this lane, where its activations and partial
// live in LDS, and whether it exists.
struct Slot {
    uint32_t op, os;   // byte offsets of row 2rp's packed indices / group scales (this lane)
    int xw, pidx;      // LDS word of this lane's activation slot; partial index of row 2rp
    bool valid;
};

// The layers of one launch: layer g owns workgroups [wg_start[g], wg_start[g + 1]), each
// with rows[g] consecutive rows of it.  NG is the capacity: single-layer launches use NG = 1,
// which keeps their kernel arguments and prologue as small as before.
template <int NG>
struct GroupTab {
    int G;
    int wg_start[NG + 1];
    int rows[NG];
    LayerDesc L[NG];
};

// XIN selects the activation input: 0 = prepared int8 x_q and s_x; 1 = fp32 and 2 = bf16
// raw activations, rotated and quantised in the prologue with the arithmetic of the
// activation kernel (every workgroup does the same, bit for bit; workgroup 0 also stores
// x_q and s_x).  SS: the group scales are staged in LDS (else each unit loads its own two
// bytes per row; used where the staging would cost rows per workgroup).
template <int MT, int XIN, int NG, bool SS>
__global__ __launch_bounds__(kThreads) void k_gemv(LinearArgs a, GroupTab<NG> gt) {
    // The pair table is a static LDS array at a compile-time address, so each lookup is one
    // v_perm for the address and one ds_read_b32; activations and partials follow it in
    // dynamic LDS.
    __shared__ __align__(16) uint32_t lds[kTabWords];
    extern __shared__ uint32_t dyn[];
    const int tid = threadIdx.x;

    // this workgroup's layer: the last one whose first workgroup is not after it (selected
    // with compile-time indices, so the table stays in kernel-argument memory)
    int gi = 0;
#pragma unroll
    for (int q = 1; q < NG; q++) gi = (q < gt.G && (int)blockIdx.x >= gt.wg_start[q]) ? q : gi;
    LayerDesc L = gt.L[0];
    int rows_per_wg = gt.rows[0], wg0 = 0;
#pragma unroll
    for (int q = 1; q < NG; q++)
        if (gi == q) {
            L = gt.L[q];
            rows_per_wg = gt.rows[q];
            wg0 = gt.wg_start[q];
        }

    const int64_t K = a.K, N = L.N;
    const int nblk = (int)(K / kRot);
    const int64_t r0 = (int64_t)((int)blockIdx.x - wg0) * rows_per_wg;
    const int nrow = (int)min((int64_t)rows_per_wg, N - r0);
    const int P = (nrow + 1) >> 1;                               // row pairs
    const int units = P * nblk;
    const int pstride = nblk | 1;                                // odd: conflict-free row sums
    const int xtok = nblk * kXBlk;                               // LDS words per token
    const uint32_t grpbytes = (uint32_t)(K / kGroup);
    uint32_t *xs = dyn;                                          // [MT][nblk][kXBlk] fp16 pairs
    uint8_t *ss = reinterpret_cast<uint8_t *>(xs + MT * xtok);   // [rows_per_wg][K/16] e4m3 scales
    float *part = reinterpret_cast<float *>(ss + (SS ? scale_lds_bytes(rows_per_wg, grpbytes) : 0));  // [MT][rows_per_wg][pstride]

    const int j = tid & 7;
    const uint32_t lanebase = (uint32_t)(tid & 63) * 4u;
    const uint32_t rowbytes = (uint32_t)(K / 2);
    // Workgroup-relative 32-bit offsets into buffer resources bounded by this workgroup's
    // rows: row 2rp+1 past the last row reads as zero and is never stored.
    const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(L.packed + r0 * rowbytes), (short)0, (int)(nrow * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(L.s_rel + r0 * grpbytes), (short)0, (int)(nrow * grpbytes), 0x00020000);
    constexpr int kNT = 2;  // non-temporal: the weights are streamed once per call

    // Units in row-major order u = rp * nblk + t; lane group g of wave w takes units
    // 8w + g + 128 i.  The wave's base unit b = 8w + 128 i is uniform: its position
    // (rpb, tb) lives in scalar registers and advances by 128 units per step; each lane
    // adds a constant delta for its g (at most one row wrap, since g % nblk < nblk).
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = (tid >> 3) & 7;
    const int gdiv = g / nblk, gmod = g - gdiv * nblk;
    const uint32_t dop = (uint32_t)gdiv * 2u * rowbytes + (uint32_t)gmod * 128u + 16u * j;
    const uint32_t dos = (uint32_t)gdiv * 2u * grpbytes + (uint32_t)gmod * 16u + 2u * j;
    const int dpidx = gdiv * 2 * pstride + gmod, dxw = gmod * kXBlk + 16 * j;
    const int sdrp = kLaneGroups / nblk, sdt = kLaneGroups - sdrp * nblk;
    int bu = 8 * wave;                       // wave base unit (uniform)
    int rpb = bu / nblk, tb = bu - rpb * nblk;
    auto make_slot = [&]() {
        Slot sl;
        const bool wrap = tb + gmod >= nblk;
        sl.valid = bu + g < units;
        const uint32_t opb = (uint32_t)rpb * 2u * rowbytes + (uint32_t)tb * 128u + dop;
        const uint32_t osb = (uint32_t)rpb * 2u * grpbytes + (uint32_t)tb * 16u + dos;
        sl.op = wrap ? opb + rowbytes : opb;   // wrap: next row pair, t - nblk
        sl.os = wrap ? osb + grpbytes : osb;
        const int pb_ = rpb * 2 * pstride + tb * 1 + dpidx, xb = tb * kXBlk + dxw;
        sl.pidx = wrap ? pb_ + 2 * pstride - nblk : pb_;
        sl.xw = wrap ? xb - nblk * kXBlk : xb;
        return sl;
    };
    auto step = [&]() {
        bu += kLaneGroups;
        tb += sdt;
        rpb += sdrp;
        if (tb >= nblk) { tb -= nblk; rpb += 1; }
    };

    // Loads are issued unconditionally (a fixed count per ring slot keeps the hardware's
    // in-order load counter exact); a unit past the end gets an offset beyond the buffer,
    // which reads as zero without touching memory.
    constexpr uint32_t kOutside = 0x80000000u;
    auto fetch = [&](const Slot &sl, u32x4 &pa, u32x4 &pb, uint32_t &sa, uint32_t &sb) {
        const uint32_t op = sl.valid ? sl.op : kOutside;
        pa = __builtin_amdgcn_raw_buffer_load_b128(rs_p, op, 0, kNT);
        pb = __builtin_amdgcn_raw_buffer_load_b128(rs_p, op + rowbytes, 0, kNT);
        if constexpr (!SS) {
            const uint32_t os = sl.valid ? sl.os : kOutside;
            sa = __builtin_amdgcn_raw_buffer_load_b16(rs_s, os, 0, kNT);
            sb = __builtin_amdgcn_raw_buffer_load_b16(rs_s, os + grpbytes, 0, kNT);
        }
    };

    // Small operands first: the row scales of this workgroup's rows (one per thread, kept
    // in a register until the final sums), and the activations.  Their loads precede the
    // weight loads in the in-order load counter, so using them does not wait for the
    // weight prefetch.
    const float sch_mine = (tid >> 3) < nrow ? L.s_ch[r0 + (tid >> 3)] : 0.0f;  // row of the first final-sum pass
    // The codebook and this wave's high-nibble level come through the scalar cache: 64
    // bytes that are the same for every lane.  As vector loads every lane would fetch the
    // whole line (64 KiB through the workgroup's load path for 64 bytes), and the table
    // build would wait, in the in-order vector load counter, behind everything issued
    // before it; scalar loads use a counter of their own.
    const __attribute__((address_space(4))) float *cbk = (const __attribute__((address_space(4))) float *)L.cb;
    float cbv[kLevels];
#pragma unroll
    for (int q = 0; q < kLevels; q++) cbv[q] = cbk[q];
    const float cb_hi = cbk[__builtin_amdgcn_readfirstlane(tid >> 6)];
    float sx_all[MT];
    const uint2 *xq8 = reinterpret_cast<const uint2 *>(a.x_q);
    const int nxc = (int)(MT * (K / 8));
    uint2 xraw[XIN == 0 ? kMaxXChunks : 1];
    // raw activations: lane row g16 (16 lanes) holds block g16 + 64 r, 16 values per lane
    float xr[XIN == 0 ? 1 : MT][kFusedRounds][16];
    const int lane64 = tid & 63, wave64 = tid >> 6;
    const int g16 = tid >> 4, t16 = tid & 15, h16 = fwht_row16_nibble(t16);
    if constexpr (XIN == 0) {
#pragma unroll
        for (int m = 0; m < MT; m++) sx_all[m] = a.s_x[m];
#pragma unroll
        for (int q = 0; q < kMaxXChunks; q++) {
            const int i = tid + q * kThreads;
            xraw[q] = i < nxc ? xq8[i] : make_uint2(0, 0);
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
            for (int r = 0; r < kFusedRounds; r++) {
                const int b = g16 + 64 * r;
                if (b < nblk) {
                    load16<XIN == 2>(a.x_raw, m * K + (int64_t)b * kRot + 16 * h16, xr[m][r]);
                } else {
#pragma unroll
                    for (int q = 0; q < 16; q++) xr[m][r][q] = 0.0f;
                }
            }
    }

    // The workgroup's group scales (nrow x K/16 contiguous bytes) are copied to LDS by the
    // buffer unit (16 bytes per lane straight into LDS, no registers), so the weight stream
    // carries no 2-byte loads.  A wave copies a 1 KiB block when its first byte is inside the
    // region; the allocation is rounded up to whole blocks.
    const int nsc = SS ? (int)(nrow * grpbytes / 16) : 0;
#pragma unroll
    for (int q = 0; q < (SS ? kScaleLoads : 0); q++) {
        const int blk = q * kThreads + 64 * wave;  // first 16-byte chunk of this wave's block
        if (blk < nsc)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_s, (__attribute__((address_space(3))) void *)(ss + 16 * blk), 16,
                16u * (uint32_t)(blk + (tid & 63)), 0, 0, kNT);
    }

    // A ring of kDepth units in flight per lane group; the first loads are issued before
    // the prologue so their HBM latency overlaps the table build.  The scheduling barrier
    // keeps every small operand's load ahead of them; with raw activations (a larger first
    // request per wave) a bare s_barrier also keeps every wave's small loads ahead of any
    // wave's weight stream.  It orders the issue only: __syncthreads() would first wait for
    // every small load to land (s_waitcnt vmcnt(0)), holding the weight stream back by a
    // whole memory round trip.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XIN != 0) __builtin_amdgcn_s_barrier();
    constexpr int kDepth = depth<MT>();
    Slot cur[kDepth];
    u32x4 pa[kDepth], pb[kDepth];
    uint32_t sa[kDepth] = {}, sb[kDepth] = {};  // per-unit scale bytes when they are not staged
#pragma unroll
    for (int d = 0; d < kDepth; d++) {
        cur[d] = make_slot();
        fetch(cur[d], pa[d], pb[d], sa[d], sb[d]);
        step();
    }

    // codebook -> fp16 pair table, scaled by 2^-ex with max |cb| = f * 2^ex, f in [0.5, 1).
    // Wave w writes entries 16w .. 16w+15 (high nibble w), each lane its own column.
    float cmax = 0.0f;
#pragma unroll
    for (int q = 0; q < kLevels; q++) cmax = fmaxf(cmax, fabsf(cbv[q]));
    int ex = 0;
    if (cmax > 0.0f) frexpf(cmax, &ex);
    const float inv = ldexpf(1.0f, -ex);
    {
        static_assert(kThreads / 64 == kLevels, "one wave per high nibble");
        const int w = tid >> 6, lane = tid & 63;
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(cb_hi * inv));
#pragma unroll
        for (int lo = 0; lo < kLevels; lo++) {
            const uint32_t v = __builtin_bit_cast(uint16_t, (_Float16)(cbv[lo] * inv)) | (hi << 16);
            lds[(16 * w + lo) * 64 + lane] = v;
        }
    }
    auto cvt2 = [](uint32_t v, int sh) {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int8_t)((v >> sh) & 0xFF)) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(int8_t)((v >> (sh + 8)) & 0xFF)) << 16);
    };
    if constexpr (XIN == 0) {
        // activations int8 -> fp16 pairs (exact), one 4-word chunk (8 values) per item, stored
        // at chunk c ^ ((j >> 1) & 3) of its 16-word lane slot j so that the 8 lanes of a group
        // reading their chunk c hit distinct banks
    #pragma unroll
        for (int q = 0; q < kMaxXChunks; q++) {
            const int i = tid + q * kThreads;
            if (i < nxc) {
                const uint2 w = xraw[q];
                const int word = 4 * i;  // logical word of this chunk (token m = word / (K/2))
                const int m = word / (int)(K / 2), wk = word - m * (int)(K / 2);
                const int d = wk & 127, lj = d >> 4, c = (d >> 2) & 3;
                const int phys = m * xtok + (wk >> 7) * kXBlk + (lj << 4) + ((c ^ xchunk_swizzle(lj, wk >> 7)) << 2);
                *reinterpret_cast<uint4 *>(xs + phys) = make_uint4(cvt2(w.x, 0), cvt2(w.x, 16), cvt2(w.y, 0), cvt2(w.y, 16));
            }
        }
    } else {
        // rotate, per-token amax over the workgroup, quantise; fp16 pairs into the swizzled
        // layout; workgroup 0 also stores x_q and s_x
        float *red = part + MT * rows_per_wg * pstride;  // [MT][16] wave maxima (dynamic LDS tail)
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < kFusedRounds; r++) {
                if (g16 + 64 * r < nblk) {  // whole 16-lane rows: absent blocks skip it
                    fwht256_row16(xr[m][r], t16);
#pragma unroll
                    for (int q = 0; q < 16; q++) amax = fmaxf(amax, fabsf(xr[m][r][q]));
                }
            }
            amax = wave_max_nonneg(amax);
            if (lane64 == 0) red[m * (kThreads / 64) + wave64] = amax;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float amax = red[m * (kThreads / 64)];
#pragma unroll
            for (int w = 1; w < kThreads / 64; w++) amax = fmaxf(amax, red[m * (kThreads / 64) + w]);
            const float sxm = amax / 127.0f;
            const float rsm = sxm >= kQuantFastMin ? 1.0f / sxm : 0.0f;
            sx_all[m] = sxm;
            if (blockIdx.x == 0 && tid == 0) a.s_x_out[m] = sxm;
#pragma unroll
            for (int r = 0; r < kFusedRounds; r++) {
                const int b = g16 + 64 * r;
                if (b < nblk) {
                    float qv[16];
                    quant16_values(xr[m][r], sxm, rsm, amax > 0.0f, qv);
                    if (blockIdx.x == 0) {
                        uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
                        for (int i = 0; i < 16; i++) wd[i >> 2] |= ((uint32_t)(int32_t)qv[i] & 0xFFu) << (8 * (i & 3));
                        reinterpret_cast<uint4 *>(a.x_q_out + m * K)[(b * kRot + 16 * h16) / 16] =
                            make_uint4(wd[0], wd[1], wd[2], wd[3]);
                    }
                    // fp16 pairs straight from the integers (exact: |q| <= 127); this lane's
                    // 16 values are logical words 8h .. 8h+7 of the block: lane slot h >> 1,
                    // chunks 2 (h & 1) and 2 (h & 1) + 1
                    uint32_t hp[8];
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        hp[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(qv[2 * i], qv[2 * i + 1]));
                    const int lj = h16 >> 1, c0 = 2 * (h16 & 1), sw = xchunk_swizzle(lj, b);
                    const int base = m * xtok + b * kXBlk + (lj << 4);
                    *reinterpret_cast<uint4 *>(xs + base + ((c0 ^ sw) << 2)) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
                    *reinterpret_cast<uint4 *>(xs + base + (((c0 + 1) ^ sw) << 2)) = make_uint4(hp[4], hp[5], hp[6], hp[7]);
                }
            }
        }
    }
    // every copy to LDS of this wave is complete once at most the ring's 2 x kDepth weight
    // loads (issued after them) are outstanding: vmcnt(2 kDepth) (gfx9 encoding, no
    // expcnt / lgkmcnt wait); the barrier then publishes them to the other waves
    static_assert(2 * depth<MT>() < 16, "vmcnt field");
    if constexpr (SS) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * depth<MT>()));
    __syncthreads();


    auto compute = [&](const Slot &sl, const u32x4 &pa, const u32x4 &pb, uint32_t sa, uint32_t sb) {
        // the two rows' scale pairs of this lane's 32 values (staged: row 2rp + 1 past the
        // last row reads stale LDS; its partial is never used)
        if constexpr (SS) {
            sa = *reinterpret_cast<const uint16_t *>(ss + sl.os);
            sb = *reinterpret_cast<const uint16_t *>(ss + sl.os + grpbytes);
        }
        const int xbase = sl.xw;
        const int xsw = xchunk_swizzle(j, xbase >> 7);
        uint32_t pair[32];
        unit_pairs(lds, lanebase, pa, pb, pair);
        // one token's activations at a time (16 registers live, whatever MT)
        float g[MT][2][2];
#pragma unroll
        for (int m = 0; m < MT; m++) {
            uint32_t xv[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint4 v = *reinterpret_cast<const uint4 *>(xs + m * xtok + xbase + 4 * (q ^ xsw));  // xbase / 128 = block
                xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y;
                xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
            }
            unit_dots(pair, xv, g[m]);
        }
        // gfx950's v_cvt_f32_fp8 decodes OCP E4M3FN (checked on all 254 finite codes)
        const float fa0 = __builtin_amdgcn_cvt_f32_fp8((int)sa, 0), fa1 = __builtin_amdgcn_cvt_f32_fp8((int)sa, 1);
        const float fb0 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0), fb1 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 1);
#pragma unroll
        for (int m = 0; m < MT; m++) {
            const float va = sum8_to_leader(fmaf(fa1, g[m][0][1], fa0 * g[m][0][0]));
            const float vb = sum8_to_leader(fmaf(fb1, g[m][1][1], fb0 * g[m][1][0]));
            if (j == 0) {
                float *pp = part + m * rows_per_wg * pstride + sl.pidx;
                pp[0] = va;
                pp[pstride] = vb;  // an odd last row pair writes row nrow < rows_per_wg, never read
            }
        }
    };

    // kDepth units went out before the prologue (they cover its latency).  The first
    // kDepth - 1 are computed as they are; from then on one unit is in flight while a unit
    // is computed: the next unit's loads are issued first, into the slot computed last.  bu
    // is the base of the next fetch, so the slot computed first in the loop body holds base
    // bu - 128.
#pragma unroll
    for (int d = 0; d + 1 < kDepth; d++)
        if (cur[d].valid) compute(cur[d], pa[d], pb[d], sa[d], sb[d]);
    while (__builtin_amdgcn_readfirstlane(bu) - kLaneGroups < units) {
#pragma unroll
        for (int d = 0; d < kDepth; d++) {
            cur[d] = make_slot();
            fetch(cur[d], pa[d], pb[d], sa[d], sb[d]);
            step();
            const int c = (d + kDepth - 1) % kDepth;
            if (cur[c].valid) compute(cur[c], pa[c], pb[c], sa[c], sb[c]);
        }
    }
    __syncthreads();

    // eight lanes per (token, row): lane e sums the row's block partials e, e + 8, ... in
    // block order, then the eight sums are added pairwise in a fixed pattern (deterministic,
    // and the same for every launch shape of the layer)
    const float cbscale = ldexpf(1.0f, ex);
    for (int i = tid >> 3; i < MT * nrow; i += kThreads / 8) {
        const int m = MT == 1 ? 0 : i / nrow, rl = i - m * nrow;
        const float *pp = part + (m * rows_per_wg + rl) * pstride;
        float acc = 0.0f;
        for (int t = j; t < nblk; t += 8) acc += pp[t];
        acc = sum8_to_leader(acc);
        if (j == 0) {
            const float sch = (i < kThreads / 8 && m == 0) ? sch_mine : L.s_ch[r0 + rl];
            const int64_t r = r0 + rl;
            float sxm = sx_all[0];
#pragma unroll
            for (int q = 1; q < MT; q++) sxm = (m == q) ? sx_all[q] : sxm;
            const float v = ((acc * sch) * sxm) * cbscale;
            if (a.y_bf16)
                static_cast<uint16_t *>(L.y)[m * N + r] = f32_to_bf16_rne(v);
            else
                static_cast<float *>(L.y)[m * N + r] = v;
        }
    }
}

// Rows per workgroup for each layer (one workgroup per CU in all, shared out in proportion
// to the layers' rows; a layer's rows per workgroup are even and small enough for its LDS),
// with or without the staged group scales.  Returns the dynamic LDS bytes, or -1.
template <int MT, int XIN, int NG>
int64_t plan_rows(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu, bool ss, GroupTab<NG> &gt) {
    const int64_t nblk = a.K / kRot;
    // dynamic part (the 64 KiB table is static): activations, staged scales, partials, then a
    // [MT][16] scratch for the fused preparation's wave maxima
    const int64_t fixed = (int64_t)MT * nblk * kXBlk * 4 + (XIN ? (int64_t)MT * (kThreads / 64) * 4 : 0);
    const int64_t dyn_max = kLdsMax - (int64_t)kTabWords * 4;
    const int64_t pstride = nblk | 1;
    const int64_t grpbytes = a.K / kGroup;
    // staged scales: at most kScaleLoads 16-byte copies per thread in all
    auto need = [&](int64_t rows) {
        return fixed + (ss ? scale_lds_bytes(rows, grpbytes) : 0) + (int64_t)MT * rows * pstride * 4;
    };
    auto fits = [&](int64_t rows) {
        return need(rows) <= dyn_max && (!ss || rows * grpbytes <= (int64_t)kScaleLoads * kThreads * 16);
    };
    int64_t total = 0;
    for (int g = 0; g < G; g++) total += layers[g].N;
    gt = GroupTab<NG>{};
    gt.G = G;
    int64_t wg = 0, max_rows = 2;
    for (int g = 0; g < G; g++) {
        const int64_t n = layers[g].N;
        int64_t want = ((int64_t)num_cu * n + total / 2) / total;
        if (want < 1) want = 1;
        int64_t rows = (n + want - 1) / want;
        rows += rows & 1;
        while (rows > 2 && !fits(rows)) rows = ((rows / 2) + 1) & ~1LL;
        if (!fits(rows)) return -1;
        gt.wg_start[g] = (int)wg;
        gt.rows[g] = (int)rows;
        gt.L[g] = layers[g];
        wg += (n + rows - 1) / rows;
        if (rows > max_rows) max_rows = rows;
    }
    gt.wg_start[G] = (int)wg;
    return need(max_rows);
}

template <int MT, int XIN, int NG, bool SS>
hipError_t launch_planned(const LinearArgs &a, const GroupTab<NG> &gt, int64_t lds, hipStream_t stream) {
    // set once per kernel instance; concurrent first calls may both set it, which is harmless
    static std::atomic<bool> attr_set{false};
    if (!attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemv<MT, XIN, NG, SS>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kLdsMax - kTabWords * 4));
        if (e != hipSuccess) return e;
        attr_set.store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((k_gemv<MT, XIN, NG, SS>), dim3((unsigned)gt.wg_start[gt.G]), dim3(kThreads), (size_t)lds, stream, a, gt);
    return hipGetLastError();
}

// The staged-scale kernel is used when staging costs no rows per workgroup (no extra
// workgroups); otherwise each unit loads its scale bytes.
template <int MT, int XIN, int NG>
hipError_t launch_mt(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu, hipStream_t stream) {
    if (G < 1 || G > NG) return hipErrorInvalidValue;
    GroupTab<NG> with{}, without{};
    const int64_t lds_with = plan_rows<MT, XIN, NG>(a, layers, G, num_cu, true, with);
    const int64_t lds_without = plan_rows<MT, XIN, NG>(a, layers, G, num_cu, false, without);
    if (lds_without < 0) return hipErrorInvalidValue;
    if (lds_with >= 0 && with.wg_start[G] <= without.wg_start[G])
        return launch_planned<MT, XIN, NG, true>(a, with, lds_with, stream);
    return launch_planned<MT, XIN, NG, false>(a, without, lds_without, stream);
}

LayerDesc single_layer(const LinearArgs &a) { return LayerDesc{a.packed, a.s_rel, a.s_ch, a.cb, a.N, a.y}; }

}  // namespace

bool gemv_supported(int64_t M, int64_t K) { return M >= 1 && M <= kMaxMT && M * K <= 40960; }

bool gemv_fused_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= 2 && K <= (int64_t)64 * kFusedRounds * kRot && gemv_supported(M, K);
}

template <int NG>
hipError_t launch_prepared(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu, hipStream_t stream) {
    switch (a.M) {
        case 1: return launch_mt<1, 0, NG>(a, layers, G, num_cu, stream);
        case 2: return launch_mt<2, 0, NG>(a, layers, G, num_cu, stream);
        case 3: return launch_mt<3, 0, NG>(a, layers, G, num_cu, stream);
        case 4: return launch_mt<4, 0, NG>(a, layers, G, num_cu, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int NG>
hipError_t launch_fused(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu, hipStream_t stream) {
    if (a.M == 1)
        return a.x_bf16 ? launch_mt<1, 2, NG>(a, layers, G, num_cu, stream) : launch_mt<1, 1, NG>(a, layers, G, num_cu, stream);
    if (a.M == 2)
        return a.x_bf16 ? launch_mt<2, 2, NG>(a, layers, G, num_cu, stream) : launch_mt<2, 1, NG>(a, layers, G, num_cu, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_multi(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu,
                             hipStream_t stream) {
    return launch_prepared<kMaxGroup>(a, layers, G, num_cu, stream);
}

hipError_t launch_gemv_fused_multi(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu,
                                   hipStream_t stream) {
    return launch_fused<kMaxGroup>(a, layers, G, num_cu, stream);
}

hipError_t launch_gemv(const LinearArgs &a, int num_cu, hipStream_t stream) {
    const LayerDesc l = single_layer(a);
    return launch_prepared<1>(a, &l, 1, num_cu, stream);
}

hipError_t launch_gemv_fused(const LinearArgs &a, int num_cu, hipStream_t stream) {
    const LayerDesc l = single_layer(a);
    return launch_fused<1>(a, &l, 1, num_cu, stream);
}

}  // namespace w4a8
