// Offline weight quantisation, entirely on the device.
//
// Model cards: "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", sections "Format" (packed
// int4 indices two per byte, an e4m3 scale per 16 values, an fp32 scale per output row, a
// 16-level per-tensor Lloyd-Max codebook fitted to the tensor's own distribution; rotation
// before quantisation, group 256) and "Reproducing" (the seed pins the codebook fit, which
// samples); "Qwen3.8-27B-W4A8 (for ComfyUI)", section "Model Overview".
//
// Steps, each a kernel on the caller's stream:
//  1. k_rotate_scale: per row, rotate every 256-block (the same lane-level transform as
//     the activation kernel), s_channel = max |w_rot|, s_rel = E4M3FN(group max / s_channel)
//     rounded to nearest even, v = w_rot / (s_channel * dec(s_rel)) -> workspace.
//  2. k_sample_keys: S = min(N*K, 2^20) fit values (all of them, or positions
//     floor(u_i * N*K / 2^64) with u_i the i-th SplitMix64 output for `seed`), as uint32
//     keys whose unsigned order is the fp32 total order (-0 before +0); padded with
//     0xFFFFFFFF to a power of two.
//  3. bitonic sort of the keys (LDS tiles of 2048 keys for the short spans).
//  4. k_prefix: running fp64 sums of the sorted values, accumulated strictly left to
//     right by one thread (the order fixes the rounding, which the codebook bits depend on).
//  5. k_lloyd: one wave runs Lloyd's iteration in fp64 from the mid-quantile start:
//     thresholds (c_j + c_{j+1}) / 2, cell bounds by binary search over the sorted values,
//     cell means from the prefix sums, at most 100 updates, stop when no bound moves;
//     codebook = (float)c.
//  6. k_assign_pack: idx = #{ j < 15 : (double)v > ((double)cb[j] + (double)cb[j+1]) / 2 },
//     two indices per byte, even element in the low nibble.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kRegBlocks = 5;
constexpr int64_t kSampleMax = 1LL << 20;
constexpr int kMaxUpdates = 100;
constexpr int kSortTile = 2048;

struct WsLayout {
    size_t v_off, keys_off, prefix_off, total;
    int64_t S, P2;
};

WsLayout layout(int64_t N, int64_t K) {
    WsLayout L{};
    const int64_t NK = N * K;
    L.S = NK < kSampleMax ? NK : kSampleMax;
    int64_t p2 = kSortTile;
    while (p2 < L.S) p2 <<= 1;
    L.P2 = p2;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.v_off = 0;
    L.keys_off = up((size_t)NK * 4);
    L.prefix_off = L.keys_off + up((size_t)L.P2 * 4);
    L.total = L.prefix_off + up((size_t)(L.S + 1) * 8);
    return L;
}

// Group scale, normalised values and the s_rel byte of one 16-group spread over 4 lanes.
__device__ __forceinline__ void scale_block(float v[4], float rmax, int lane, float *vout,
                                            uint8_t *srel_out) {
    float g = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    g = fmaxf(g, __shfl_xor(g, 1));
    g = fmaxf(g, __shfl_xor(g, 2));
    const uint32_t code = (rmax > 0.0f) ? f32_to_e4m3_rne(g / rmax) : 0u;
    const float d = rmax * e4m3_to_f32(code);
    float4 o;
    o.x = (d > 0.0f) ? v[0] / d : 0.0f;
    o.y = (d > 0.0f) ? v[1] / d : 0.0f;
    o.z = (d > 0.0f) ? v[2] / d : 0.0f;
    o.w = (d > 0.0f) ? v[3] / d : 0.0f;
    *reinterpret_cast<float4 *>(vout + 4 * lane) = o;
    if ((lane & 3) == 0) srel_out[lane >> 2] = (uint8_t)code;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_rotate_scale(const void *__restrict__ w, int64_t K,
                                                           float *__restrict__ vout,
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
            if (b < nblk) scale_block(keep[i], rmax, lane, vout + row + (int64_t)b * kRot, srow + b * 16);
        }
    } else {
        for (int b = wave; b < nblk; b += kWaves) {
            float v[4];
            load4<BF16>(w, row + (int64_t)b * kRot + 4 * lane, v);
            fwht256_lane4(v, lane);
            scale_block(v, rmax, lane, vout + row + (int64_t)b * kRot, srow + b * 16);
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

__global__ void k_sample_keys(const float *__restrict__ v, int64_t NK, int64_t S, int64_t P2,
                              uint64_t seed, uint32_t *__restrict__ keys) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= P2) return;
    uint32_t key = 0xFFFFFFFFu;
    if (i < S) {
        int64_t pos = i;
        if (NK > kSampleMax) pos = (int64_t)__umul64hi(splitmix64_at(seed, (uint64_t)i), (uint64_t)NK);
        key = f32_to_key(v[pos]);
    }
    keys[i] = key;
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

// Running fp64 sums P[0] = 0, P[i+1] = P[i] + value(i), strictly in index order.
__global__ __launch_bounds__(256) void k_prefix(const uint32_t *__restrict__ keys, int64_t S,
                                                double *__restrict__ P) {
    constexpr int kChunk = 4096;
    __shared__ double buf[kChunk];
    double run = 0.0;
    if (threadIdx.x == 0) P[0] = 0.0;
    for (int64_t c0 = 0; c0 < S; c0 += kChunk) {
        const int n = (int)((S - c0) < kChunk ? (S - c0) : kChunk);
        for (int i = threadIdx.x; i < n; i += blockDim.x) buf[i] = (double)key_to_f32(keys[c0 + i]);
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 0; i < n; i++) {
                run = run + buf[i];
                P[c0 + i + 1] = run;
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ int64_t count_le(const uint32_t *keys, int64_t S, double t) {
    int64_t lo = 0, hi = S;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if ((double)key_to_f32(keys[mid]) <= t) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(64) void k_lloyd(const uint32_t *__restrict__ keys,
                                              const double *__restrict__ P, int64_t S,
                                              float *__restrict__ cb) {
    __shared__ double c[kLevels];
    __shared__ int64_t b[kLevels + 1], prev[kLevels + 1];
    __shared__ int changed;
    const int j = threadIdx.x;
    if (j < kLevels) c[j] = (double)key_to_f32(keys[((int64_t)(2 * j + 1) * S) / 32]);
    if (j <= kLevels) prev[j] = -1;
    __syncthreads();
    int updates = 0;
    for (int pass = 0; pass <= kMaxUpdates; pass++) {
        if (j == 0) { b[0] = 0; b[kLevels] = S; changed = 0; }
        if (j < kLevels - 1) b[j + 1] = count_le(keys, S, (c[j] + c[j + 1]) / 2.0);
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

__global__ void k_assign_pack(const float *__restrict__ v, int64_t half_nk,
                              const float *__restrict__ cb, int8_t *__restrict__ packed) {
    __shared__ double mid[kLevels - 1];
    if (threadIdx.x < kLevels - 1)
        mid[threadIdx.x] = ((double)cb[threadIdx.x] + (double)cb[threadIdx.x + 1]) / 2.0;
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= half_nk) return;
    const float2 p = reinterpret_cast<const float2 *>(v)[i];
    const double x0 = p.x, x1 = p.y;
    int i0 = 0, i1 = 0;
#pragma unroll
    for (int j = 0; j < kLevels - 1; j++) {
        i0 += (x0 > mid[j]) ? 1 : 0;
        i1 += (x1 > mid[j]) ? 1 : 0;
    }
    packed[i] = (int8_t)(uint8_t)(i0 | (i1 << 4));
}

}  // namespace

size_t quantize_workspace_bytes(int64_t N, int64_t K) { return layout(N, K).total; }

hipError_t launch_quantize(const void *w, int w_bf16, int64_t N, int64_t K, uint64_t seed,
                           int8_t *packed, uint8_t *s_rel, float *s_ch, float *cb,
                           void *workspace, hipStream_t stream) {
    const WsLayout L = layout(N, K);
    char *ws = static_cast<char *>(workspace);
    float *v = reinterpret_cast<float *>(ws + L.v_off);
    uint32_t *keys = reinterpret_cast<uint32_t *>(ws + L.keys_off);
    double *P = reinterpret_cast<double *>(ws + L.prefix_off);
    const int64_t NK = N * K;
    hipError_t e;

    if (w_bf16)
        hipLaunchKernelGGL(k_rotate_scale<true>, dim3((unsigned)N), dim3(kThreads), 0, stream, w, K, v, s_rel, s_ch);
    else
        hipLaunchKernelGGL(k_rotate_scale<false>, dim3((unsigned)N), dim3(kThreads), 0, stream, w, K, v, s_rel, s_ch);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    hipLaunchKernelGGL(k_sample_keys, dim3((unsigned)((L.P2 + 255) / 256)), dim3(256), 0, stream, v, NK, L.S,
                       L.P2, seed, keys);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const unsigned tiles = (unsigned)(L.P2 / kSortTile);
    hipLaunchKernelGGL(k_bitonic_tile, dim3(tiles), dim3(kSortTile / 2), 0, stream, keys, (int64_t)2,
                       (int64_t)kSortTile);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int64_t k = 2 * kSortTile; k <= L.P2; k <<= 1) {
        for (int64_t j = k >> 1; j >= kSortTile; j >>= 1) {  // spans the tiles cannot hold
            const int64_t pairs = L.P2 / 2;
            hipLaunchKernelGGL(k_bitonic_global, dim3((unsigned)(pairs / 256)), dim3(256), 0, stream, keys, k, j);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_bitonic_tile, dim3(tiles), dim3(kSortTile / 2), 0, stream, keys, k, k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    hipLaunchKernelGGL(k_prefix, dim3(1), dim3(256), 0, stream, keys, L.S, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_lloyd, dim3(1), dim3(64), 0, stream, keys, P, L.S, cb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t half_nk = NK / 2;
    hipLaunchKernelGGL(k_assign_pack, dim3((unsigned)((half_nk + 255) / 256)), dim3(256), 0, stream, v, half_nk,
                       cb, packed);
    return hipGetLastError();
}

}  // namespace w4a8
