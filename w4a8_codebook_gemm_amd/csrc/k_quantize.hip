// Offline weight quantisation, entirely on the device.
//
// Model cards: "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", sections "Format" (packed
// int4 indices two per byte, an e4m3 scale per 16 values, an fp32 scale per output row, a
// 16-level per-tensor Lloyd-Max codebook fitted to the tensor's own distribution; rotation
// before quantisation, group 256) and "Reproducing" (the seed pins the codebook fit, which
// samples); "Qwen3.8-27B-W4A8 (for ComfyUI)", section "Model Overview".
//
// Steps, each a kernel (or a few) on the caller's stream:
//  1. k_rotate_scale16 (k_rotate_scale for rows over 128 blocks): per row, rotate every
//     256-block, s_channel = max |w_rot|, s_rel = E4M3FN(group max / s_channel) rounded to
//     nearest even.  The row transform runs each block on a 16-lane DPP row; it matches the
//     lane transform bit for bit except for the sign of an exact zero, which maxima of |v|
//     do not see.
//  2. Sampling: S = min(N*K, 2^20) fit values v = w_rot / (s_channel * dec(s_rel)) -- all of
//     them (k_sample_keys), or those at positions floor(u_i * N*K / 2^64) with u_i the i-th
//     SplitMix64 output for `seed` (k_sample_count / _scan_* / _list / _blocks: the samples
//     bucketed by block, each block rotated once) -- as uint32 keys whose unsigned order is
//     the fp32 total order (-0 before +0); padded with 0xFFFFFFFF to a power of two.  The
//     values come from the lane transform (the sign of a zero can reach a codebook level),
//     and are never stored beyond the sample: the workspace holds only the sample and its
//     prefix sums, at most 12 MiB whatever N and K.
//  3. sort of the keys: a full 2^20-key sample by an LSD radix sort (four stable passes of
//     8-bit digits), smaller ones by a bitonic network (LDS tiles of 2048 keys for the short
//     spans, up to three of the longer passes per sweep).
//  4. k_prefix_*: running fp64 sums of the sorted values in the blocked order (blocks of
//     kPrefixBlock values summed left to right from 0, the block offsets left to right over
//     the block totals, then offset + block-local sum; the order fixes the rounding, which
//     the codebook bits depend on).  One lane per block, so 1024 blocks run at once.
//  5. k_lloyd: one workgroup runs Lloyd's iteration in fp64 from the mid-quantile start:
//     thresholds (c_j + c_{j+1}) / 2, cell bounds by search over the sorted values, cell
//     means from the prefix sums, at most 100 updates, stop when no bound moves;
//     codebook = (float)c.
//  6. k_assign_pack: per block (row transform, as in step 1), normalise again,
//     idx = #{ j < 15 : (double)v > ((double)cb[j] + (double)cb[j+1]) / 2 } (decided by an
//     equivalent fp32 compare), two indices per byte, even element in the low nibble.
#include <atomic>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kRegBlocks = 5;
constexpr int64_t kSampleMax = 1LL << 20;
constexpr int kMaxUpdates = 100;
constexpr int kSortTile = 2048;

constexpr size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr int64_t pow2_at_least(int64_t s) {
    int64_t p = kSortTile;
    while (p < s) p <<= 1;
    return p;
}

// Workspace: the sample keys (padded to a power of two) and their fp64 prefix sums.
struct WsLayout {
    size_t keys_off, prefix_off, total;
    int64_t S, P2;
};

constexpr WsLayout layout_for_sample(int64_t S) {
    WsLayout L{};
    L.S = S;
    L.P2 = pow2_at_least(S);
    L.keys_off = 0;
    L.prefix_off = round256((size_t)L.P2 * 4);
    L.total = L.prefix_off + round256((size_t)(L.S + 1) * 8);
    return L;
}

WsLayout layout(int64_t N, int64_t K) {
    const int64_t NK = N * K;
    return layout_for_sample(NK < kSampleMax ? NK : kSampleMax);
}

// The largest workspace any shape needs (a full 2^20-value sample): the size of the
// no-allocation entry point's static scratch.
constexpr size_t kScratchBytes = layout_for_sample(kSampleMax).total;

// The group-scale code of one 16-group spread over 4 lanes (rotated values v, row max rmax).
__device__ __forceinline__ uint32_t group_code(const float v[4], float rmax) {
    float g = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    g = fmaxf(g, __shfl_xor(g, 1));
    g = fmaxf(g, __shfl_xor(g, 2));
    return (rmax > 0.0f) ? f32_to_e4m3_rne(g / rmax) : 0u;
}

// Normalised values v / (rmax * dec(code)), 0 where that product is 0.
__device__ __forceinline__ void normalise4(float v[4], float rmax, uint32_t code) {
    const float d = rmax * e4m3_to_f32(code);
#pragma unroll
    for (int q = 0; q < 4; q++) v[q] = (d > 0.0f) ? v[q] / d : 0.0f;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_rotate_scale(const void *__restrict__ w, int64_t K,
                                                           uint8_t *__restrict__ s_rel,
                                                           float *__restrict__ s_ch) {
    __shared__ float red[kWaves];
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = (int)(K / kRot);
    const int64_t row = r * K;
    const bool in_regs = nblk <= kWaves * kRegBlocks;
    float keep[kRegBlocks][4];
    float amax = 0.0f;
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kRegBlocks; i++) {
            const int b = wave + i * kWaves;
            if (b < nblk) {
                load4<BF16>(w, row + (int64_t)b * kRot + 4 * lane, keep[i]);
                fwht256_lane4(keep[i], lane);
#pragma unroll
                for (int q = 0; q < 4; q++) amax = fmaxf(amax, fabsf(keep[i][q]));
            }
        }
    } else {
        for (int b = wave; b < nblk; b += kWaves) {
            float v[4];
            load4<BF16>(w, row + (int64_t)b * kRot + 4 * lane, v);
            fwht256_lane4(v, lane);
#pragma unroll
            for (int q = 0; q < 4; q++) amax = fmaxf(amax, fabsf(v[q]));
        }
    }
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    float rmax = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; i++) rmax = fmaxf(rmax, red[i]);
    if (threadIdx.x == 0) s_ch[r] = rmax;
    uint8_t *srow = s_rel + r * (K / kGroup);
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kRegBlocks; i++) {
            const int b = wave + i * kWaves;
            if (b < nblk) {
                const uint32_t code = group_code(keep[i], rmax);
                if ((lane & 3) == 0) srow[b * 16 + (lane >> 2)] = (uint8_t)code;
            }
        }
    } else {
        for (int b = wave; b < nblk; b += kWaves) {
            float v[4];
            load4<BF16>(w, row + (int64_t)b * kRot + 4 * lane, v);
            fwht256_lane4(v, lane);
            const uint32_t code = group_code(v, rmax);
            if ((lane & 3) == 0) srow[b * 16 + (lane >> 2)] = (uint8_t)code;
        }
    }
}

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t f32_to_key(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// One wave per job.  Sampled (N*K > 2^20): job i is sample i, the value at position
// floor(u_i * N*K / 2^64); every value (N*K <= 2^20): job i is 256-block i, whose values are
// samples 256 i .. 256 i + 255 in position order.  Either way the wave rotates the whole
// 256-block (lane l holds elements 4l .. 4l+3) and normalises with the row's s_channel and
// the group's s_rel, as k_rotate_scale derived them.  Threads past the last job pad the
// keys from S to P2.
constexpr int kSampleWaves = 4;

template <bool BF16>
__global__ __launch_bounds__(64 * kSampleWaves) void k_sample_keys(
    const void *__restrict__ w, int64_t K, int64_t NK, int64_t S, int64_t P2, uint64_t seed,
    const float *__restrict__ s_ch, const uint8_t *__restrict__ s_rel, uint32_t *__restrict__ keys) {
    const int lane = threadIdx.x & 63;
    const int64_t job = (int64_t)blockIdx.x * kSampleWaves + (threadIdx.x >> 6);
    const bool sampled = NK > kSampleMax;
    const int64_t jobs = sampled ? S : NK / kRot;
    if (job < jobs) {
        int64_t pos = job * kRot;
        if (sampled) pos = (int64_t)__umul64hi(splitmix64_at(seed, (uint64_t)job), (uint64_t)NK);
        const int64_t r = pos / K, blk0 = (pos - r * K) / kRot * kRot;   // first element of the block
        float v[4];
        load4<BF16>(w, r * K + blk0 + 4 * lane, v);
        fwht256_lane4(v, lane);
        const uint32_t code = s_rel[r * (K / kGroup) + blk0 / kGroup + (lane >> 2)];
        normalise4(v, s_ch[r], code);
        if (sampled) {
            const int e = (int)(pos - r * K - blk0);                     // the sample's element
            if ((e >> 2) == lane) keys[job] = f32_to_key(v[e & 3]);
        } else {
            uint4 k4 = make_uint4(f32_to_key(v[0]), f32_to_key(v[1]), f32_to_key(v[2]), f32_to_key(v[3]));
            *reinterpret_cast<uint4 *>(keys + job * kRot + 4 * lane) = k4;
        }
    }
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = S + t; i < P2; i += nthreads) keys[i] = 0xFFFFFFFFu;
}

// Step 1 on 16-lane DPP rows for rows of up to 2 x 64 blocks: lane row g rotates blocks g and
// g + (lane rows) with the row transform (bit-identical to the lane transform up to the sign
// of a zero, which neither maximum sees), so that each lane holds one whole group of 16: its
// group maximum needs no exchange.  The row maximum goes through the waves' maxima in LDS.
template <bool BF16, int R>
__global__ __launch_bounds__(1024) void k_rotate_scale16(const void *__restrict__ w, int64_t K,
                                                         uint8_t *__restrict__ s_rel, float *__restrict__ s_ch) {
    __shared__ float red[16];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const int rows16 = blockDim.x >> 4, g = tid >> 4, t16 = tid & 15, h = fwht_row16_nibble(t16);
    const int nblk = (int)(K / kRot);
    float v[R][16];
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < R; q++) {
        const int b = g + q * rows16;
        // an absent block re-reads the last one (all 16 lanes of its row alike) and is ignored
        load16<BF16>(w, r * K + (int64_t)(b < nblk ? b : nblk - 1) * kRot + 16 * h, v[q]);
    }
#pragma unroll
    for (int q = 0; q < R; q++) {
        fwht256_row16(v[q], t16);
        if (g + q * rows16 < nblk)
#pragma unroll
            for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(v[q][i]));
    }
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
    if ((tid & 63) == 0) red[wave] = amax;
    __syncthreads();
    float rmax = red[0];
    for (int i = 1; i < nwaves; i++) rmax = fmaxf(rmax, red[i]);
    if (tid == 0) s_ch[r] = rmax;
#pragma unroll
    for (int q = 0; q < R; q++) {
        const int b = g + q * rows16;
        if (b < nblk) {
            float gm = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; i++) gm = fmaxf(gm, fabsf(v[q][i]));
            s_rel[r * (K / kGroup) + b * 16 + h] = (uint8_t)((rmax > 0.0f) ? f32_to_e4m3_rne(gm / rmax) : 0u);
        }
    }
}

// Sampled fits (N*K > 2^20) by block: k_sample_keys rotates a whole 256-block for every
// sample, about three times per block at the MLP shapes.  These kernels rotate each block
// that holds samples once instead.  For a chunk of kChunkBlocks 256-blocks at a time they
// count the samples per block (each sample parking its rank within its block), turn the
// counts into offsets, list each block's sample indices at offset + rank (any order within
// a block) and let a wave rotate each block and write keys[i] for each of its samples i --
// the same keys at the same places as k_sample_keys writes.  The counts and the list live
// in the prefix-sum area of the workspace, unused until the sort is done.
constexpr int64_t kChunkBlocks = (1 << 19) - 1024;   // blocks per pass; the scratch below fits the prefix area
constexpr int kCountThreads = 256;

__device__ __forceinline__ int64_t sample_pos(uint64_t seed, int64_t i, int64_t NK) {
    return (int64_t)__umul64hi(splitmix64_at(seed, (uint64_t)i), (uint64_t)NK);
}

__global__ __launch_bounds__(kCountThreads) void k_fill_u32(uint32_t *__restrict__ p, int64_t n, uint32_t v) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = t; i < n; i += stride) p[i] = v;
}

// Counts the samples per block; each sample of the chunk parks its rank within its block
// in keys[i] (that key is written only later, by k_sample_blocks).
__global__ __launch_bounds__(kCountThreads) void k_sample_count(uint64_t seed, int64_t S, int64_t NK, int64_t c0,
                                                                int64_t c1, uint32_t *__restrict__ cnt,
                                                                uint32_t *__restrict__ keys) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= S) return;
    const int64_t blk = sample_pos(seed, i, NK) / kRot;
    if (blk >= c0 && blk < c1) keys[i] = atomicAdd(&cnt[blk - c0], 1u);
}

// cnt[0 .. n) -> exclusive offsets (integers: exact in any order), cnt[n] = total.  Segments
// of 1024 counts: each workgroup scans its own in LDS and records the segment's total; then
// each adds the totals of the segments before it.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_sample_scan_seg(uint32_t *__restrict__ cnt, int64_t n,
                                                                  uint32_t *__restrict__ segsum) {
    __shared__ uint32_t sh[kScanThreads];
    const int t = threadIdx.x;
    const int64_t i = (int64_t)blockIdx.x * kScanThreads + t;
    const uint32_t v = i < n ? cnt[i] : 0u;
    sh[t] = v;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
        const uint32_t x = t >= d ? sh[t - d] : 0u;
        __syncthreads();
        sh[t] += x;
        __syncthreads();
    }
    if (i < n) cnt[i] = sh[t] - v;
    if (t == kScanThreads - 1) segsum[blockIdx.x] = sh[t];
}

__global__ __launch_bounds__(kScanThreads) void k_sample_scan_add(uint32_t *__restrict__ cnt, int64_t n,
                                                                  const uint32_t *__restrict__ segsum) {
    __shared__ uint32_t base;
    const int t = threadIdx.x;
    const int seg = blockIdx.x;
    if (t == 0) base = 0u;
    __syncthreads();
    for (int q = t; q < seg; q += kScanThreads) atomicAdd(&base, segsum[q]);
    __syncthreads();
    const uint32_t b = base;
    const int64_t i = (int64_t)seg * kScanThreads + t;
    if (i < n) cnt[i] += b;
    if (seg == (int)gridDim.x - 1 && t == 0) cnt[n] = b + segsum[seg];
}

// Lists each block's samples at its offset plus the rank k_sample_count parked.
__global__ __launch_bounds__(kCountThreads) void k_sample_list(uint64_t seed, int64_t S, int64_t NK, int64_t c0,
                                                               int64_t c1, const uint32_t *__restrict__ off,
                                                               const uint32_t *__restrict__ keys,
                                                               uint32_t *__restrict__ list) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= S) return;
    const int64_t blk = sample_pos(seed, i, NK) / kRot;
    if (blk >= c0 && blk < c1) list[off[blk - c0] + keys[i]] = (uint32_t)i;
}

// Four blocks of the chunk per wave: rotate and normalise each as k_sample_keys does, then
// write the key of each sample it holds.  Every block's loads and sample counts go out
// first, then the first 64 listed samples of every block (lane t takes the t-th), so a wave
// waits for memory twice for its four blocks; each sample's value comes from the lane that
// holds it.
constexpr int kSampleNB = 4;
template <bool BF16>
__global__ __launch_bounds__(64 * kSampleWaves) void k_sample_blocks(
    const void *__restrict__ w, int64_t K, int64_t NK, uint64_t seed, int64_t c0, int64_t c1,
    const float *__restrict__ s_ch, const uint8_t *__restrict__ s_rel, const uint32_t *__restrict__ cnt,
    const uint32_t *__restrict__ list, uint32_t *__restrict__ keys) {
    const int lane = threadIdx.x & 63;
    const int64_t first = c0 + ((int64_t)blockIdx.x * kSampleWaves + (threadIdx.x >> 6)) * kSampleNB;
    if (first >= c1) return;
    float v[kSampleNB][4], rmax[kSampleNB];
    uint32_t code[kSampleNB], q0[kSampleNB], q1[kSampleNB];
    int64_t pos0[kSampleNB];
#pragma unroll
    for (int b = 0; b < kSampleNB; b++) {
        const int64_t blk = first + b < c1 ? first + b : first;   // past the chunk: a copy of the first, no samples
        pos0[b] = blk * kRot;
        const int64_t r = pos0[b] / K, blk0 = pos0[b] - r * K;
        load4<BF16>(w, pos0[b] + 4 * lane, v[b]);
        code[b] = s_rel[r * (K / kGroup) + blk0 / kGroup + (lane >> 2)];
        rmax[b] = s_ch[r];
        q0[b] = cnt[blk - c0];
        q1[b] = first + b < c1 ? cnt[blk - c0 + 1] : q0[b];
    }
    uint32_t li[kSampleNB];
#pragma unroll
    for (int b = 0; b < kSampleNB; b++) {
        const uint32_t q = q0[b] + (uint32_t)lane;
        li[b] = list[q < q1[b] ? q : 0u];   // entry 0 is in the list's storage whatever the count
    }
#pragma unroll
    for (int b = 0; b < kSampleNB; b++) {
        fwht256_lane4(v[b], lane);
        normalise4(v[b], rmax[b], code[b]);
    }
#pragma unroll
    for (int b = 0; b < kSampleNB; b++) {
        for (uint32_t qb = q0[b]; qb < q1[b]; qb += 64) {
            const uint32_t q = qb + (uint32_t)lane;
            const bool mine = q < q1[b];
            const int64_t i = !mine ? 0 : (qb == q0[b] ? (int64_t)li[b] : (int64_t)list[q]);
            const int e = mine ? (int)(sample_pos(seed, i, NK) - pos0[b]) : 0;   // the sample's element
            const int src = e >> 2;
            const float a0 = __shfl(v[b][0], src), a1 = __shfl(v[b][1], src), a2 = __shfl(v[b][2], src),
                        a3 = __shfl(v[b][3], src);
            const int c = e & 3;
            const float val = c == 0 ? a0 : c == 1 ? a1 : c == 2 ? a2 : a3;
            if (mine) keys[i] = f32_to_key(val);
        }
    }
}

// Bitonic network: pass (k, j) compares i with i ^ j, ascending where (i & k) == 0.
__device__ __forceinline__ void cmp_swap(uint32_t &x, uint32_t &y, bool asc) {
    if ((x > y) == asc) {
        const uint32_t t = x;
        x = y;
        y = t;
    }
}

__global__ void k_bitonic_global(uint32_t *keys, int64_t k, int64_t j) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one pair per thread
    const int64_t i = (t / j) * 2 * j + (t % j);
    const int64_t l = i + j;
    uint32_t x = keys[i], y = keys[l];
    cmp_swap(x, y, (i & k) == 0);
    keys[i] = x;
    keys[l] = y;
}

// Passes (k, j) and (k, j / 2) in one sweep: thread t owns i (bits j and j / 2 clear) and
// i + j / 2, i + j, i + 3 j / 2, which those two passes compare only among themselves, all
// in one direction (k > j).
__global__ void k_bitonic_global2(uint32_t *keys, int64_t k, int64_t j) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t h = j >> 1;
    const int64_t i = (t / h) * 2 * j + (t % h);
    uint32_t a = keys[i], b = keys[i + h], c = keys[i + j], d = keys[i + j + h];
    const bool asc = (i & k) == 0;
    cmp_swap(a, c, asc);
    cmp_swap(b, d, asc);
    cmp_swap(a, b, asc);
    cmp_swap(c, d, asc);
    keys[i] = a;
    keys[i + h] = b;
    keys[i + j] = c;
    keys[i + j + h] = d;
}

// Passes (k, j), (k, j / 2) and (k, j / 4) in one sweep: thread t owns the eight elements
// i + m j / 4 (m = 0 .. 7, i with bits j, j / 2, j / 4 clear), which those passes compare
// only among themselves.
__global__ void k_bitonic_global3(uint32_t *keys, int64_t k, int64_t j) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t q = j >> 2;
    const int64_t i = (t / q) * 2 * j + (t % q);
    uint32_t x[8];
#pragma unroll
    for (int m = 0; m < 8; m++) x[m] = keys[i + m * q];
    const bool asc = (i & k) == 0;
#pragma unroll
    for (int m = 0; m < 4; m++) cmp_swap(x[m], x[m + 4], asc);
#pragma unroll
    for (int m = 0; m < 8; m += 4) {
        cmp_swap(x[m], x[m + 2], asc);
        cmp_swap(x[m + 1], x[m + 3], asc);
    }
#pragma unroll
    for (int m = 0; m < 8; m += 2) cmp_swap(x[m], x[m + 1], asc);
#pragma unroll
    for (int m = 0; m < 8; m++) keys[i + m * q] = x[m];
}

// All passes with j < kSortTile for one k (k_from == k_to), or the whole sort of every
// tile up to k = kSortTile (k_from = 2, k_to = kSortTile), inside one LDS tile.
__global__ __launch_bounds__(kSortTile / 2) void k_bitonic_tile(uint32_t *keys, int64_t k_from,
                                                                int64_t k_to) {
    __shared__ uint32_t s[kSortTile];
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    const int t = threadIdx.x;
    s[t] = keys[base + t];
    s[t + kSortTile / 2] = keys[base + t + kSortTile / 2];
    __syncthreads();
    for (int64_t k = k_from; k <= k_to; k <<= 1) {
        for (int64_t j = (k >> 1) < kSortTile / 2 ? (k >> 1) : kSortTile / 2; j > 0; j >>= 1) {
            const int i = (int)((t / j) * 2 * j + (t % j));
            const int l = i + (int)j;
            uint32_t x = s[i], y = s[l];
            cmp_swap(x, y, ((base + i) & k) == 0);
            s[i] = x;
            s[l] = y;
            __syncthreads();
        }
    }
    keys[base + t] = s[t];
    keys[base + t + kSortTile / 2] = s[t + kSortTile / 2];
}

// LSD radix sort of a full 2^20-key sample (S = P2): four stable passes of 8-bit digits,
// ping-ponging between the keys and a copy in the prefix-sum area (idle until the sort is
// done).  Per pass: each 1024-key tile counts its digits (k_radix_hist, digit-major
// counts), the counts are scanned into offsets (k_sample_scan_*), and each tile writes its
// keys to offset + rank, the rank counting the equal digits before the key in the tile:
// wave ballots over the digit's bits find the equal lanes, per-wave counts in LDS order the
// waves and rounds.  The sorted keys are the bitonic network's, key for key.
constexpr int kRadixTile = 1024;
constexpr int kRadixThreads = 256;

__global__ __launch_bounds__(kRadixThreads) void k_radix_hist(const uint32_t *__restrict__ in, int shift, int ntiles,
                                                              uint32_t *__restrict__ hist) {
    __shared__ uint32_t h[256];
    const int t = threadIdx.x;
    h[t] = 0u;
    __syncthreads();
    const uint32_t *tile = in + (int64_t)blockIdx.x * kRadixTile;
#pragma unroll
    for (int q = 0; q < kRadixTile / kRadixThreads; q++) atomicAdd(&h[(tile[q * kRadixThreads + t] >> shift) & 255u], 1u);
    __syncthreads();
    hist[(int64_t)t * ntiles + blockIdx.x] = h[t];
}

__global__ __launch_bounds__(kRadixThreads) void k_radix_scatter(const uint32_t *__restrict__ in,
                                                                 uint32_t *__restrict__ out, int shift, int ntiles,
                                                                 const uint32_t *__restrict__ off) {
    __shared__ uint32_t run[256];                        // keys of each digit in earlier rounds
    __shared__ uint32_t wcnt[kRadixThreads / 64][256];   // this round's count per wave and digit
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    run[t] = 0u;
    const uint32_t *tile = in + (int64_t)blockIdx.x * kRadixTile;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int round = 0; round < kRadixTile / kRadixThreads; round++) {
#pragma unroll
        for (int w = 0; w < kRadixThreads / 64; w++) wcnt[w][t] = 0u;
        const uint32_t key = tile[round * kRadixThreads + t];
        const uint32_t d = (key >> shift) & 255u;
        unsigned long long peers = ~0ull;
#pragma unroll
        for (int bit = 0; bit < 8; bit++) {
            const unsigned long long m = __ballot((d >> bit) & 1u);
            peers &= ((d >> bit) & 1u) ? m : ~m;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & below);
        __syncthreads();   // the counts are zeroed
        if (rank == 0) wcnt[wave][d] = (uint32_t)__popcll(peers);   // the lowest lane of its digit
        __syncthreads();
        uint32_t pre = run[d];
        for (int w = 0; w < wave; w++) pre += wcnt[w][d];
        out[off[(int64_t)d * ntiles + blockIdx.x] + pre + rank] = key;
        __syncthreads();   // every lane has read run and wcnt
        uint32_t add = 0u;
#pragma unroll
        for (int w = 0; w < kRadixThreads / 64; w++) add += wcnt[w][t];
        run[t] += add;
        __syncthreads();
    }
}

// Running fp64 sums P[0] = 0, P[i+1] = P[i] + value(i), strictly in index order.
constexpr int kPrefixBlock = 1024;
constexpr int kPrefixThreads = (int)(kSampleMax / kPrefixBlock);  // one lane per block

// One lane's pass over its block [b0, b1): the left-to-right fp64 chain from 0; with
// WRITE, P[i + 1] = off + (chain up to i).  The keys come 16 bytes per load, the next 32
// values requested while the current 32 are summed (the prefetch address is clamped to the
// block, so every load is issued on every path).
template <bool WRITE>
__device__ __forceinline__ double prefix_pass(const uint32_t *__restrict__ keys, int64_t b0, int64_t b1,
                                              double off, double *__restrict__ P) {
    constexpr int kG = 32;
    double run = 0.0;
    const int64_t nfull = b0 + ((b1 - b0) / kG) * kG;
    const uint4 *k4 = reinterpret_cast<const uint4 *>(keys);  // b0 is a multiple of 1024
    uint4 cur[kG / 4], nxt[kG / 4];
    const int64_t first = b0 < nfull ? b0 : 0;
#pragma unroll
    for (int q = 0; q < kG / 4; q++) cur[q] = k4[first / 4 + q];
    for (int64_t i = b0; i < nfull; i += kG) {
        const int64_t j = i + kG < nfull ? i + kG : i;
#pragma unroll
        for (int q = 0; q < kG / 4; q++) nxt[q] = k4[j / 4 + q];
#pragma unroll
        for (int k = 0; k < kG; k++) {
            const uint4 w = cur[k >> 2];
            const uint32_t key = (k & 3) == 0 ? w.x : (k & 3) == 1 ? w.y : (k & 3) == 2 ? w.z : w.w;
            run = run + (double)key_to_f32(key);
            if (WRITE) P[i + k + 1] = off + run;
        }
#pragma unroll
        for (int q = 0; q < kG / 4; q++) cur[q] = nxt[q];
    }
    for (int64_t i = nfull; i < b1; i++) {
        run = run + (double)key_to_f32(keys[i]);
        if (WRITE) P[i + 1] = off + run;
    }
    return run;
}

// P[0] = 0; P[i + 1] = off[b] + (s[b0] + ... + s[i]) for i in block b = [b0, b0 + 1024),
// the block-local sum running left to right from 0 and off[b] = tot[0] + ... + tot[b - 1]
// running left to right from 0 over the block totals.  Three launches, one lane per block
// in one-wave workgroups (so the 1024 chains spread over 16 compute units instead of
// sharing one): the block totals, parked in P[b0 + 1]; the offsets, which replace them
// there; then each lane's outputs.  Each lane runs its block's chain twice (once for the
// total, once for the outputs) rather than storing and re-reading it.  A block holds at
// least one value, so P[b0 + 1] exists; only lane b reads or writes it in the last launch.
constexpr int kPrefixWave = 64;
__global__ __launch_bounds__(kPrefixWave) void k_prefix_tot(const uint32_t *__restrict__ keys, int64_t S,
                                                            double *__restrict__ P) {
    const int b = blockIdx.x * kPrefixWave + threadIdx.x;
    const int nb = (int)((S + kPrefixBlock - 1) / kPrefixBlock);
    if (b >= nb) return;
    const int64_t b0 = (int64_t)b * kPrefixBlock;
    const int64_t b1 = b0 + kPrefixBlock < S ? b0 + kPrefixBlock : S;
    P[b0 + 1] = prefix_pass<false>(keys, b0, b1, 0.0, P);
}

__global__ __launch_bounds__(kPrefixThreads) void k_prefix_offs(int64_t S, double *__restrict__ P) {
    __shared__ double tot[kPrefixThreads];
    const int t = threadIdx.x;
    const int nb = (int)((S + kPrefixBlock - 1) / kPrefixBlock);
    if (t < nb) tot[t] = P[(int64_t)t * kPrefixBlock + 1];
    __syncthreads();
    if (t == 0) {
        double off = 0.0;
        for (int b = 0; b < nb; b++) {
            const double tb = tot[b];
            tot[b] = off;
            off = off + tb;
        }
    }
    __syncthreads();
    if (t < nb) P[(int64_t)t * kPrefixBlock + 1] = tot[t];
}

__global__ __launch_bounds__(kPrefixWave) void k_prefix_write(const uint32_t *__restrict__ keys, int64_t S,
                                                              double *__restrict__ P) {
    const int b = blockIdx.x * kPrefixWave + threadIdx.x;
    const int nb = (int)((S + kPrefixBlock - 1) / kPrefixBlock);
    if (b >= nb) return;
    const int64_t b0 = (int64_t)b * kPrefixBlock;
    const int64_t b1 = b0 + kPrefixBlock < S ? b0 + kPrefixBlock : S;
    const double off = P[b0 + 1];
    if (b == 0) P[0] = 0.0;
    prefix_pass<true>(keys, b0, b1, off, P);
}

// Lloyd's cell bounds: the number of sorted values <= t, found by the 16 lanes of one
// group per threshold.  A 16-way search over an LDS copy of every 32nd value (each lane
// tests one of 16 evenly spaced entries; the group's ballot tells which sixteenth holds the
// boundary) finds the 32-value window that holds it; the window (one 128-byte line, two
// values per lane) is then counted by a ballot.  The count, and so every bound, is the one
// a search over all the values gives.
constexpr int kIndexStride = 32;
constexpr int kIndexMax = (int)(kSampleMax / kIndexStride);   // 128 KiB of fp32
constexpr int kLloydThreads = 256;                              // 16 lanes per threshold

__device__ __forceinline__ uint32_t group16_count(bool pred, int lane) {
    const unsigned long long m = __ballot(pred);
    return (uint32_t)__popcll((m >> (16 * (lane >> 4))) & 0xFFFFull);
}

__device__ __forceinline__ int64_t count_le16(const float *idx, int ni, const uint32_t *keys, int64_t S, double t,
                                              int lane) {
    const int sl = lane & 15;
    // c = #{entries <= t} stays in [lo, hi]
    int lo = 0, hi = ni;
    while (lo < hi) {   // the same bounds in all 16 lanes of the group
        const int n = hi - lo;
        const int p = lo + (int)(((int64_t)(sl + 1) * n + 15) / 16) - 1;   // lo <= p <= hi - 1
        const uint32_t k = group16_count((double)idx[p] <= t, lane);
        const int pk1 = lo + (int)(((int64_t)k * n + 15) / 16) - 1;        // pivot k - 1
        const int pk = lo + (int)(((int64_t)(k + 1) * n + 15) / 16) - 1;   // pivot k
        if (k == 0) {
            hi = pk;
        } else {
            lo = pk1 + 1;
            if (k < 16) hi = pk;
        }
    }
    if (lo == 0) return 0;   // the smallest value is above t
    // values before 32 (lo - 1) are <= t and values from 32 lo on (if any) above it; the
    // window [32 (lo - 1), 32 lo) lies inside the keys, whose length is a multiple of 32
    const int64_t base = (int64_t)(lo - 1) * kIndexStride;
    const uint2 w2 = reinterpret_cast<const uint2 *>(keys + base)[sl];
    const bool p0 = base + 2 * sl < S && (double)key_to_f32(w2.x) <= t;
    const bool p1 = base + 2 * sl + 1 < S && (double)key_to_f32(w2.y) <= t;
    return base + group16_count(p0, lane) + group16_count(p1, lane);
}

__global__ __launch_bounds__(kLloydThreads) void k_lloyd(const uint32_t *__restrict__ keys,
                                                         const double *__restrict__ P, int64_t S,
                                                         float *__restrict__ cb) {
    __shared__ float idx[kIndexMax];
    __shared__ double c[kLevels];
    __shared__ int64_t b[kLevels + 1], prev[kLevels + 1];
    __shared__ int changed;
    const int j = threadIdx.x;
    const int ni = (int)((S + kIndexStride - 1) / kIndexStride);
    for (int q = j; q < ni; q += kLloydThreads) idx[q] = key_to_f32(keys[(int64_t)q * kIndexStride]);
    if (j < kLevels) c[j] = (double)key_to_f32(keys[((int64_t)(2 * j + 1) * S) / 32]);
    if (j <= kLevels) prev[j] = -1;
    __syncthreads();
    int updates = 0;
    for (int pass = 0; pass <= kMaxUpdates; pass++) {
        if (j == 0) { b[0] = 0; b[kLevels] = S; changed = 0; }
        {
            // group g = j / 16 searches threshold g (group 15 repeats threshold 14 and drops it)
            const int g = j >> 4, gt = g < kLevels - 1 ? g : kLevels - 2;
            const int64_t n = count_le16(idx, ni, keys, S, (c[gt] + c[gt + 1]) / 2.0, j & 63);
            if (g < kLevels - 1 && (j & 15) == 0) b[g + 1] = n;
        }
        __syncthreads();
        if (j <= kLevels && b[j] != prev[j]) changed = 1;
        __syncthreads();
        if (!changed || updates == kMaxUpdates) break;
        if (j < kLevels) {
            const int64_t n = b[j + 1] - b[j];
            if (n > 0) c[j] = (P[b[j + 1]] - P[b[j]]) / (double)n;
        }
        if (j <= kLevels) prev[j] = b[j];
        updates++;
        __syncthreads();
    }
    if (j < kLevels) cb[j] = (float)c[j];
}

// Per 256-block on one 16-lane DPP row (four blocks per wave, 16 per workgroup): rotate it
// again with the row transform (bit-identical to the lane transform of steps 1 and 2 up to
// the sign of a zero, which no output depends on), so that each lane holds one whole group of
// 16 values; normalise, take each value's nearest level and store the lane's 16 indices as 8
// bytes, two per byte.
constexpr int kAssignThreads = 256;
template <bool BF16>
__global__ __launch_bounds__(kAssignThreads) void k_assign_pack(const void *__restrict__ w, int64_t N, int64_t K,
                                                                const float *__restrict__ s_ch,
                                                                const uint8_t *__restrict__ s_rel,
                                                                const float *__restrict__ cb,
                                                                int8_t *__restrict__ packed) {
    // each midpoint (cb[j] + cb[j+1]) / 2, exact in fp64, as the largest fp32 at or below it:
    // for an fp32 v, (double)v > mid exactly when v > that fp32, so one fp32 compare per
    // level decides what the fp64 compare decides
    __shared__ float thr[kLevels - 1];
    if (threadIdx.x < kLevels - 1) {
        const double m = ((double)cb[threadIdx.x] + (double)cb[threadIdx.x + 1]) / 2.0;
        float f = (float)m;
        if ((double)f > m) f = nextafterf(f, -INFINITY);
        thr[threadIdx.x] = f;
    }
    __syncthreads();
    const int t16 = threadIdx.x & 15, h = fwht_row16_nibble(t16);
    const int64_t nblk = K / kRot;
    const int64_t gb = (int64_t)blockIdx.x * (kAssignThreads / 16) + (threadIdx.x >> 4);
    const bool live = gb < N * nblk;   // the same for the 16 lanes of a row
    const int64_t g0 = live ? gb : 0;
    const int64_t r = g0 / nblk, b = g0 - r * nblk;
    float v[16];
    load16<BF16>(w, r * K + b * kRot + 16 * h, v);
    fwht256_row16(v, t16);
    const float d = s_ch[r] * e4m3_to_f32(s_rel[r * (K / kGroup) + b * 16 + h]);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 16; q++) {
        const float x = (d > 0.0f) ? v[q] / d : 0.0f;
        // the number of thresholds below x, by a four-step binary search over the ascending
        // thresholds (the same count as comparing with all fifteen)
        int idx = 0;
#pragma unroll
        for (int step = 8; step >= 1; step >>= 1) idx += (x > thr[idx + step - 1]) ? step : 0;
        if (q < 8) lo |= (uint32_t)idx << (4 * q);
        else hi |= (uint32_t)idx << (4 * (q - 8));
    }
    if (live) *reinterpret_cast<uint2 *>(packed + r * (K / 2) + b * (kRot / 2) + 8 * h) = make_uint2(lo, hi);
}

// Scratch of the no-allocation entry point: one array per device, as large as the largest
// workspace (12,583,168 bytes), held by every device the library runs on until the process
// ends.  In host code its name stands for the host-side shadow only; kernels get the device
// address that hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];

}  // namespace

size_t quantize_workspace_bytes(int64_t N, int64_t K) { return layout(N, K).total; }

hipError_t quantize_scratch(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // with this device current: its own copy of the array (two threads may both look it
        // up; they store the same address)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    *bytes = kScratchBytes;
    return hipSuccess;
}

hipError_t launch_quantize(const void *w, int w_bf16, int64_t N, int64_t K, uint64_t seed,
                           int8_t *packed, uint8_t *s_rel, float *s_ch, float *cb,
                           void *workspace, hipStream_t stream) {
    const WsLayout L = layout(N, K);
    char *ws = static_cast<char *>(workspace);
    uint32_t *keys = reinterpret_cast<uint32_t *>(ws + L.keys_off);
    double *P = reinterpret_cast<double *>(ws + L.prefix_off);
    const int64_t NK = N * K;
    hipError_t e;

    const int64_t nblk = K / kRot;
    if (nblk <= 128) {
        // 16 lanes per block, whole waves, one or two rounds
        const int rounds = nblk <= 64 ? 1 : 2;
        const unsigned threads = (unsigned)(((nblk + rounds - 1) / rounds * 16 + 63) / 64 * 64);
        if (rounds == 1) {
            if (w_bf16)
                hipLaunchKernelGGL((k_rotate_scale16<true, 1>), dim3((unsigned)N), dim3(threads), 0, stream, w, K, s_rel, s_ch);
            else
                hipLaunchKernelGGL((k_rotate_scale16<false, 1>), dim3((unsigned)N), dim3(threads), 0, stream, w, K, s_rel, s_ch);
        } else {
            if (w_bf16)
                hipLaunchKernelGGL((k_rotate_scale16<true, 2>), dim3((unsigned)N), dim3(threads), 0, stream, w, K, s_rel, s_ch);
            else
                hipLaunchKernelGGL((k_rotate_scale16<false, 2>), dim3((unsigned)N), dim3(threads), 0, stream, w, K, s_rel, s_ch);
        }
    } else if (w_bf16) {
        hipLaunchKernelGGL(k_rotate_scale<true>, dim3((unsigned)N), dim3(kThreads), 0, stream, w, K, s_rel, s_ch);
    } else {
        hipLaunchKernelGGL(k_rotate_scale<false>, dim3((unsigned)N), dim3(kThreads), 0, stream, w, K, s_rel, s_ch);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    if (NK > kSampleMax) {
        // S = 2^20 = P2: no padding.  Counts and the list in the prefix-sum area.
        static_assert(round256((kChunkBlocks + 1) * 4) + kSampleMax * 4 +
                              4 * ((kChunkBlocks + kScanThreads - 1) / kScanThreads) <=
                          round256((kSampleMax + 1) * 8),
                      "sampling scratch inside the prefix area");
        uint32_t *cnt = reinterpret_cast<uint32_t *>(P);
        uint32_t *list = cnt + round256((kChunkBlocks + 1) * 4) / 4;
        uint32_t *segsum = list + kSampleMax;
        const int64_t nb = NK / kRot;
        const unsigned cgrid = (unsigned)((L.S + kCountThreads - 1) / kCountThreads);
        for (int64_t c0 = 0; c0 < nb; c0 += kChunkBlocks) {
            const int64_t c1 = c0 + kChunkBlocks < nb ? c0 + kChunkBlocks : nb;
            hipLaunchKernelGGL(k_fill_u32, dim3(256), dim3(kCountThreads), 0, stream, cnt, c1 - c0 + 1, 0u);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_sample_count, dim3(cgrid), dim3(kCountThreads), 0, stream, seed, L.S, NK, c0, c1, cnt,
                               keys);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const unsigned nseg = (unsigned)((c1 - c0 + kScanThreads - 1) / kScanThreads);
            hipLaunchKernelGGL(k_sample_scan_seg, dim3(nseg), dim3(kScanThreads), 0, stream, cnt, c1 - c0, segsum);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_sample_scan_add, dim3(nseg), dim3(kScanThreads), 0, stream, cnt, c1 - c0, segsum);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_sample_list, dim3(cgrid), dim3(kCountThreads), 0, stream, seed, L.S, NK, c0, c1, cnt,
                               keys, list);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const unsigned bgrid = (unsigned)((c1 - c0 + kSampleWaves * kSampleNB - 1) / (kSampleWaves * kSampleNB));
            if (w_bf16)
                hipLaunchKernelGGL(k_sample_blocks<true>, dim3(bgrid), dim3(64 * kSampleWaves), 0, stream, w, K, NK,
                                   seed, c0, c1, s_ch, s_rel, cnt, list, keys);
            else
                hipLaunchKernelGGL(k_sample_blocks<false>, dim3(bgrid), dim3(64 * kSampleWaves), 0, stream, w, K, NK,
                                   seed, c0, c1, s_ch, s_rel, cnt, list, keys);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        const int64_t jobs = NK / kRot;
        const unsigned sblocks = (unsigned)((jobs + kSampleWaves - 1) / kSampleWaves);
        if (w_bf16)
            hipLaunchKernelGGL(k_sample_keys<true>, dim3(sblocks), dim3(64 * kSampleWaves), 0, stream, w, K, NK, L.S,
                               L.P2, seed, s_ch, s_rel, keys);
        else
            hipLaunchKernelGGL(k_sample_keys<false>, dim3(sblocks), dim3(64 * kSampleWaves), 0, stream, w, K, NK, L.S,
                               L.P2, seed, s_ch, s_rel, keys);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    if (L.S == kSampleMax) {
        // radix passes: keys -> copy -> keys -> copy -> keys, in the prefix-sum area the copy,
        // the digit counts (+ their total) and the scan's segment totals
        const int ntiles = (int)(kSampleMax / kRadixTile);
        const int64_t ncnt = (int64_t)256 * ntiles;
        static_assert(kSampleMax * 4 + round256(((size_t)256 * (kSampleMax / kRadixTile) + 1) * 4) +
                              4 * ((256 * (kSampleMax / kRadixTile) + kScanThreads - 1) / kScanThreads) <=
                          round256((kSampleMax + 1) * 8),
                      "radix scratch inside the prefix area");
        uint32_t *copy = reinterpret_cast<uint32_t *>(P);
        uint32_t *hist = copy + kSampleMax;
        uint32_t *segsum = hist + round256((size_t)(ncnt + 1) * 4) / 4;
        const unsigned nseg = (unsigned)((ncnt + kScanThreads - 1) / kScanThreads);
        for (int pass = 0; pass < 4; pass++) {
            const uint32_t *in = (pass & 1) ? copy : keys;
            uint32_t *out = (pass & 1) ? keys : copy;
            hipLaunchKernelGGL(k_radix_hist, dim3(ntiles), dim3(kRadixThreads), 0, stream, in, 8 * pass, ntiles, hist);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_sample_scan_seg, dim3(nseg), dim3(kScanThreads), 0, stream, hist, ncnt, segsum);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_sample_scan_add, dim3(nseg), dim3(kScanThreads), 0, stream, hist, ncnt, segsum);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(k_radix_scatter, dim3(ntiles), dim3(kRadixThreads), 0, stream, in, out, 8 * pass, ntiles,
                               hist);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
    const unsigned tiles = (unsigned)(L.P2 / kSortTile);
    hipLaunchKernelGGL(k_bitonic_tile, dim3(tiles), dim3(kSortTile / 2), 0, stream, keys, (int64_t)2,
                       (int64_t)kSortTile);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int64_t k = 2 * kSortTile; k <= L.P2; k <<= 1) {
        for (int64_t j = k >> 1; j >= kSortTile;) {  // spans the tiles cannot hold, up to three at a time
            if ((j >> 2) >= kSortTile) {
                hipLaunchKernelGGL(k_bitonic_global3, dim3((unsigned)(L.P2 / 8 / 256)), dim3(256), 0, stream, keys, k, j);
                j >>= 3;
            } else if ((j >> 1) >= kSortTile) {
                hipLaunchKernelGGL(k_bitonic_global2, dim3((unsigned)(L.P2 / 4 / 256)), dim3(256), 0, stream, keys, k, j);
                j >>= 2;
            } else {
                hipLaunchKernelGGL(k_bitonic_global, dim3((unsigned)(L.P2 / 2 / 256)), dim3(256), 0, stream, keys, k, j);
                j >>= 1;
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_bitonic_tile, dim3(tiles), dim3(kSortTile / 2), 0, stream, keys, k, k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    }

    const unsigned pblocks = (unsigned)((L.S + (int64_t)kPrefixBlock * kPrefixWave - 1) / ((int64_t)kPrefixBlock * kPrefixWave));
    hipLaunchKernelGGL(k_prefix_tot, dim3(pblocks), dim3(kPrefixWave), 0, stream, keys, L.S, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefix_offs, dim3(1), dim3(kPrefixThreads), 0, stream, L.S, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefix_write, dim3(pblocks), dim3(kPrefixWave), 0, stream, keys, L.S, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_lloyd, dim3(1), dim3(kLloydThreads), 0, stream, keys, P, L.S, cb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned ablocks = (unsigned)((NK / kRot + kAssignThreads / 16 - 1) / (kAssignThreads / 16));
    if (w_bf16)
        hipLaunchKernelGGL(k_assign_pack<true>, dim3(ablocks), dim3(kAssignThreads), 0, stream, w, N, K, s_ch, s_rel,
                           cb, packed);
    else
        hipLaunchKernelGGL(k_assign_pack<false>, dim3(ablocks), dim3(kAssignThreads), 0, stream, w, N, K, s_ch, s_rel,
                           cb, packed);
    return hipGetLastError();
}

}  // namespace w4a8
