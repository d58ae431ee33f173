// Internal declarations of the gfx950 W4A8 library: launchers and small device helpers.
// Not part of the public ABI (include/w4a8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

constexpr int kRot = 256;    // rotation block along K
constexpr int kGroup = 16;   // values per fp8 group scale
constexpr int kLevels = 16;  // codebook levels

// ---------------------------------------------------------------- e4m3 (OCP E4M3FN)
// Decode by bit assembly: a normal code (e > 0) is the fp32 with exponent e - 7 + 127 and
// the 3 mantissa bits on top of the fp32 mantissa; a subnormal code m * 2^-9 is formed as
// (1 + m/8) * 2^-6 - 2^-6, exact in fp32.  NaN codes are outside the format's use.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t mag = (c & 0x7Fu) << 20;
    float normal = __uint_as_float(mag + 0x3C000000u);
    float sub = __uint_as_float(mag + 0x3C800000u) - 0x1p-6f;
    float v = (c & 0x78u) ? normal : sub;
    return (c & 0x80u) ? -v : v;
}

// Round a non-negative finite fp32 to the nearest E4M3FN code, ties to the even code,
// saturating at 448 (0x7E).  Works on the bit pattern: pick the code exponent, then round
// the fp32 mantissa to 3 bits (subnormal codes use a fixed 2^-9 quantum).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float x) {
    if (!(x > 0.0f)) return 0u;              // 0 (and -0)
    if (x >= 464.0f) return 0x7Eu;           // beyond the 448/480 midpoint: saturate
    uint32_t b = __float_as_uint(x);
    int e = (int)(b >> 23) - 127;            // unbiased fp32 exponent (x normal here or tiny)
    if (e < -6) {                            // code subnormal range: value = m * 2^-9
        float q = x * 0x1p9f;                // exact scaling by a power of two
        float r = rintf(q);                  // ties to even
        return (uint32_t)r;                  // 0..8; 8 == 2^-6 is the first normal code 0x08
    }
    uint32_t mant = b & 0x7FFFFFu;
    uint32_t keep = mant >> 20;              // top 3 mantissa bits
    uint32_t rest = mant & 0xFFFFFu;         // 20 discarded bits
    uint32_t half = 0x80000u;
    uint32_t up = (rest > half) || (rest == half && (keep & 1u));
    uint32_t code = ((uint32_t)(e + 7) << 3) + keep + up;  // carry into the exponent is right
    return code > 0x7Eu ? 0x7Eu : code;
}

// In-place rotation of one 256-block held as 4 consecutive elements per lane of a wave
// (lane l holds elements 4l..4l+3).  Spans 1 and 2 are in-lane; spans 4..128 exchange with
// lane ^ 1 .. lane ^ 32.  Each butterfly is one fp32 add (lower element) and one fp32
// subtract (upper element = lower - upper) in the fixed span order 1, 2, ..., 128; the
// x 1/16 is exact.  Must be called by all 64 lanes of the wave.
__device__ __forceinline__ void fwht256_lane4(float v[4], int lane) {
    // span 1: pairs (0,1), (2,3)
    float a0 = v[0] + v[1], a1 = v[0] - v[1];
    float a2 = v[2] + v[3], a3 = v[2] - v[3];
    // span 2: pairs (0,2), (1,3)
    v[0] = a0 + a2; v[2] = a0 - a2;
    v[1] = a1 + a3; v[3] = a1 - a3;
    // spans 4..128: partner lane = lane ^ s; the lower lane keeps a + b, the upper a - b
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const bool upper = (lane & s) != 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            float other = __shfl_xor(v[q], s);
            v[q] = upper ? (other - v[q]) : (v[q] + other);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; q++) v[q] = v[q] * 0.0625f;
}

// The same rotation of one 256-block on the 16 lanes of a DPP row, 16 values per lane, with
// no LDS traffic.  Element bits 0..3 index the lane's registers (v[j] = element 16h + j), so
// spans 1..8 are in-lane; element bits 4..7 (the "high nibble" h) are spread over the row's
// lanes as h = t ^ 3*bit2(t) for row position t.  Under that map, flipping element bit 4, 5,
// 6 or 7 is lane xor 1, 2, 7 or 8: the DPP patterns quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror and row_ror:8, each a single exchange within the row.
// A cross-lane butterfly is one fma with the partner's value as the DPP operand,
// fma(partner, +-1, own): the lower lane gets RN(upper + lower) and the upper lane
// RN(upper - lower), the negation of the subtraction's rounded result.  Each value is thus
// held with the sign (-1)^(number of stages in which its lane was the upper one), that is
// (-1)^popcount(h) at the end, which the final exact scaling by +-1/16 removes: the result
// is bit-identical to the add/subtract order above (a zero may come out as -0).  Every lane
// of the row must execute it.
__device__ __forceinline__ int fwht_row16_nibble(int t) { return t ^ (((t >> 2) & 1) * 3); }

// One cross-lane stage: sixteen v_fmac_f32 with the DPP pattern on the multiplicand.  The
// s_nop covers the two wait states a DPP read needs after the VALU write of its source.
#define W4A8_FMAC_DPP16(PAT)                                                                        \
    asm volatile("s_nop 1\n"                                                                      \
                 "v_fmac_f32_dpp %0, %0, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %1, %1, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %2, %2, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %3, %3, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %4, %4, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %5, %5, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %6, %6, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %7, %7, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %8, %8, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %9, %9, %16 " PAT " row_mask:0xf bank_mask:0xf\n"                 \
                 "v_fmac_f32_dpp %10, %10, %16 " PAT " row_mask:0xf bank_mask:0xf\n"               \
                 "v_fmac_f32_dpp %11, %11, %16 " PAT " row_mask:0xf bank_mask:0xf\n"               \
                 "v_fmac_f32_dpp %12, %12, %16 " PAT " row_mask:0xf bank_mask:0xf\n"               \
                 "v_fmac_f32_dpp %13, %13, %16 " PAT " row_mask:0xf bank_mask:0xf\n"               \
                 "v_fmac_f32_dpp %14, %14, %16 " PAT " row_mask:0xf bank_mask:0xf\n"               \
                 "v_fmac_f32_dpp %15, %15, %16 " PAT " row_mask:0xf bank_mask:0xf\n"               \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),        \
                   "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),      \
                   "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                              \
                 : "v"(sgn))

__device__ __forceinline__ void fwht_row16_stage_xor1(float v[16], float sgn) { W4A8_FMAC_DPP16("quad_perm:[1,0,3,2]"); }
__device__ __forceinline__ void fwht_row16_stage_xor2(float v[16], float sgn) { W4A8_FMAC_DPP16("quad_perm:[2,3,0,1]"); }
__device__ __forceinline__ void fwht_row16_stage_mirror(float v[16], float sgn) { W4A8_FMAC_DPP16("row_half_mirror"); }
__device__ __forceinline__ void fwht_row16_stage_ror8(float v[16], float sgn) { W4A8_FMAC_DPP16("row_ror:8"); }
#undef W4A8_FMAC_DPP16

__device__ __forceinline__ void fwht256_row16(float v[16], int t) {
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if (i & s) continue;
            const float a = v[i], b = v[i + s];
            v[i] = a + b;
            v[i + s] = a - b;
        }
    }
    const int h = fwht_row16_nibble(t);
    fwht_row16_stage_xor1(v, (h & 1) ? -1.0f : 1.0f);    // span 16:  lane ^ 1
    fwht_row16_stage_xor2(v, (h & 2) ? -1.0f : 1.0f);    // span 32:  lane ^ 2
    fwht_row16_stage_mirror(v, (h & 4) ? -1.0f : 1.0f);  // span 64:  lane ^ 7 (half mirror)
    fwht_row16_stage_ror8(v, (h & 8) ? -1.0f : 1.0f);    // span 128: lane ^ 8 (rotate by 8)
    const float scale = (__builtin_popcount(h) & 1) ? -0.0625f : 0.0625f;
#pragma unroll
    for (int q = 0; q < 16; q++) v[q] = v[q] * scale;
}

// Sixteen consecutive activations (fp32, or bf16 widened exactly) starting at element off
// (a multiple of 16).
template <bool BF16>
__device__ __forceinline__ void load16(const void *x, int64_t off, float v[16]) {
    if constexpr (BF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
        const uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float4 f = p[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
    }
}

// Four consecutive activations (fp32, or bf16 widened exactly) starting at element off.
template <bool BF16>
__device__ __forceinline__ void load4(const void *x, int64_t off, float v[4]) {
    if constexpr (BF16) {
        uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + off);
        v[0] = __uint_as_float(u.x << 16);
        v[1] = __uint_as_float(u.x & 0xFFFF0000u);
        v[2] = __uint_as_float(u.y << 16);
        v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
        float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
}

// Per-token symmetric int8 of four rotated values with scale s = amax / 127 (s > 0): IEEE
// division, round to nearest even, clamp to +-127; packed little-endian into one word.
__device__ __forceinline__ uint32_t quant4(const float v[4], float s) {
    uint32_t out = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        float r = rintf(v[q] / s);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        out |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * q);
    }
    return out;
}

// quant4 over sixteen values -> sixteen int8 bytes.
__device__ __forceinline__ uint4 quant16(const float v[16], float s) {
    return make_uint4(quant4(v, s), quant4(v + 4, s), quant4(v + 8, s), quant4(v + 12, s));
}

// The same bytes with the IEEE quotient v / s formed from r = RN(1 / s) by Markstein's
// correction: q0 = RN(v r), e = fma(-q0, s, v) (exact), q = fma(e, r, q0) = RN(v / s)
// (P. Markstein, "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990).  The theorem needs r correctly rounded and no
// overflow or underflow in the steps: callers use it for s >= kQuantFastMin only (then
// |v / s| <= 127 and r < 2^100; quotients that underflow are far below 1/2 and round to 0
// either way).  Checked against IEEE division around every rounding boundary.
constexpr float kQuantFastMin = 0x1p-100f;
__device__ __forceinline__ uint32_t quant4_r(const float v[4], float s, float r) {
    uint32_t out = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const float q0 = v[q] * r;
        const float e = fmaf(-q0, s, v[q]);
        float t = rintf(fmaf(e, r, q0));
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        out |= ((uint32_t)(int32_t)t & 0xFFu) << (8 * q);
    }
    return out;
}

// quant16 choosing the exact fast path when the scale allows it (uniform per token).
__device__ __forceinline__ uint4 quant16_auto(const float v[16], float s, float r) {
    if (s >= kQuantFastMin)
        return make_uint4(quant4_r(v, s, r), quant4_r(v + 4, s, r), quant4_r(v + 8, s, r), quant4_r(v + 12, s, r));
    return quant16(v, s);
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// ---------------------------------------------------------------- int8 level tables
// Sixteen int8 levels, one per 4-bit index, looked up with byte permutes.
struct CbI8 {
    uint32_t t[4];  // the 16 levels as bytes, level j in byte j % 4 of t[j / 4]
};

// four 4-bit indices (one per byte) -> the four int8 levels
__device__ __forceinline__ uint32_t lookup4(const CbI8 &c, uint32_t idx4) {
    const uint32_t sel = idx4 & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(c.t[1], c.t[0], sel);
    const uint32_t hi = __builtin_amdgcn_perm(c.t[3], c.t[2], sel);
    const uint32_t msel = ((idx4 >> 3) & 0x01010101u) | 0x0C0C0C0Cu;  // 0x0C -> 0x00, 0x0D -> 0xFF
    const uint32_t mask = __builtin_amdgcn_perm(0u, 0u, msel);
    return (mask & hi) | (~mask & lo);
}

// one packed dword (k = 0..7: low nibble of byte b is k = 2b) -> 8 int8 in k order
__device__ __forceinline__ uint2 decode8(const CbI8 &c, uint32_t w) {
    const uint32_t even = lookup4(c, w & 0x0F0F0F0Fu);         // k = 0, 2, 4, 6
    const uint32_t odd = lookup4(c, (w >> 4) & 0x0F0F0F0Fu);   // k = 1, 3, 5, 7
    return make_uint2(__builtin_amdgcn_perm(odd, even, 0x05010400u), __builtin_amdgcn_perm(odd, even, 0x07030602u));
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Shapes were validated by the caller.
hipError_t launch_prepare(const void *x, int x_bf16, int64_t M, int64_t K, int8_t *x_q,
                          float *s_x, int num_cu, hipStream_t stream);

struct LinearArgs {
    const int8_t *x_q;
    const float *s_x;
    int64_t M, K, N;
    const int8_t *packed;
    const uint8_t *s_rel;
    const float *s_ch;
    const float *cb;
    void *y;
    int y_bf16;
    // fused activation preparation (w4a8_forward): raw activations in, x_q / s_x out
    const void *x_raw;
    int x_bf16;
    int8_t *x_q_out;
    float *s_x_out;
    // batched decode with K split into ksplit parts: the parts' sums [ksplit][M][N] and one
    // arrival counter per row block (zero between calls)
    float *ws_part = nullptr;
    uint32_t *ws_cnt = nullptr;
    int ksplit = 1;
};

bool gemv_supported(int64_t M, int64_t K);
bool gemv_fused_supported(int64_t M, int64_t K);
hipError_t launch_gemv(const LinearArgs &a, int num_cu, hipStream_t stream);
hipError_t launch_gemv_fused(const LinearArgs &a, int num_cu, hipStream_t stream);

// Several layers that read the same activations, run by one GEMV launch: the persistent
// workgroups are split between the layers in proportion to their rows.  The activation
// fields of LinearArgs apply to all of them; its layer fields are ignored.
constexpr int kMaxGroup = 8;
struct LayerDesc {
    const int8_t *packed;
    const uint8_t *s_rel;
    const float *s_ch;
    const float *cb;
    int64_t N;
    void *y;
};
hipError_t launch_gemv_multi(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu,
                             hipStream_t stream);
hipError_t launch_gemv_fused_multi(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu,
                                   hipStream_t stream);
// the decoded-weight GEMM on the int8 and the fp16 form of the codebook
hipError_t launch_gemm_i8(const LinearArgs &a, hipStream_t stream);
hipError_t launch_gemm_f16(const LinearArgs &a, hipStream_t stream);
// int8 MFMA, exact int32 partial per group of 16, fp32 fold on the vector ALU
hipError_t launch_gemm_i8_fold(const LinearArgs &a, hipStream_t stream);
// whether its tile count for (M, N) fits the grid
bool gemm_dec_tiles_fit(int64_t M, int64_t N);
bool gemm_rq_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_rq(const LinearArgs &a, hipStream_t stream);
bool skinny_supported(int64_t M, int64_t N, int64_t K);
constexpr int64_t kSkinnyCounterBytes = 4096;  // the split's arrival counters: 1024 row blocks
int skinny_split(int64_t M, int64_t N, int64_t K, int num_cu);
int64_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int num_cu);
hipError_t launch_gemm_skinny(const LinearArgs &a, int num_cu, hipStream_t stream);
// G layers of a.N rows each in one launch (no K split), every output bit-identical to the
// single-layer launch's
hipError_t launch_gemm_skinny_multi(const LinearArgs &a, const LayerDesc *layers, int G, int num_cu,
                                    hipStream_t stream);

// W8A8 comparator (per-row int8 weights of the rotated rows, no codebook)
struct W8Args {
    const int8_t *x_q;
    const float *s_x;
    int64_t M, K, N;
    const int8_t *w_q;
    const float *s_w;
    void *y;
    int y_bf16;
};
constexpr int64_t kW8GemvMaxX = 65536;   // M*K activation bytes the decode GEMV stages in LDS
constexpr int64_t kW8MaxK = 131072;      // exact int32 sums: 127^2 * K < 2^31
bool w8_gemv_supported(int64_t M, int64_t K);
hipError_t launch_w8_gemv(const W8Args &a, int num_cu, hipStream_t stream);
hipError_t launch_w8_gemm(const W8Args &a, hipStream_t stream);

size_t quantize_workspace_bytes(int64_t N, int64_t K);
// The no-allocation entry point's scratch on the current device: its device address and
// size (the first call on a device looks the address up).
hipError_t quantize_scratch(void **ptr, size_t *bytes);
hipError_t launch_quantize(const void *w, int w_bf16, int64_t N, int64_t K, uint64_t seed,
                           int8_t *packed, uint8_t *s_rel, float *s_ch, float *cb,
                           void *workspace, hipStream_t stream);

}  // namespace w4a8
