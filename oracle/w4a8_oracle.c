/*
 * CPU oracle for the asym_w4a8_int8 ("ConvRot") W4A8 codebook linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant generator with the HIP library; nothing in the product path may call it.
 *
 * It is a plain, slow, obviously correct statement of what the layer computes, written
 * from two model cards:
 *   [card A] "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI" -- sections "Why this exists",
 *            "Format", "Verification", "Reproducing";
 *   [card B] "Qwen3.8-27B-W4A8 (for ComfyUI)" -- sections "Model Overview", "Accuracy".
 * Where the cards leave a step open, the reading taken is stated at the function.
 *
 * Layout (row-major, contiguous):
 *   W        fp32   [N][K]      weights, out x in
 *   packed   int8   [N][K/2]    4-bit codebook indices, element 2j in the low nibble
 *   s_rel    uint8  [N][K/16]   e4m3 (OCP E4M3FN) bit patterns, one per 16 values
 *   s_ch     fp32   [N]         per-row scale
 *   cb       fp32   [16]        per-tensor codebook, ascending
 *   x        fp32   [M][K]      activations; x_q int8 [M][K]; s_x fp32 [M]
 *
 * Build flags (see oracle/build.py): -O2 -ffp-contract=off -fno-fast-math, so every
 * fp32 operation below is one IEEE-754 round-to-nearest-even operation.
 *
 * Parity pins for every function live in tests/test_oracle.py.  None is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ROT 256  /* rotation block along in_features  [card A "Format"; card B "Model Overview"] */
#define GRP 16   /* values per group scale             [card A "Format"; card B "Model Overview"] */
#define LEVELS 16
#define FIT_SAMPLE_MAX (1LL << 20)
#define FIT_MAX_ITERS 100

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------------------
 * Rotation.  [card A "Format": a group-wise Hadamard rotation before quantisation,
 * rotation group 256; card B "Model Overview": Hadamard rotation in 256-blocks.]
 * Reading: Sylvester Hadamard of order 256 in natural order, scaled by 1/16 so it is
 * orthonormal and its own inverse.  Computed as the fast transform with stages
 * h = 1, 2, 4, ..., 128 in that order, each butterfly (a, b) -> (a + b, a - b) one fp32
 * add and one fp32 subtract, and the 1/16 applied last (exact: a power of two).
 * Result: v[j] = (1/16) sum_i (-1)^popcount(i & j) v_in[i], up to the rounding of the
 * adds.  The stage order is fixed because the int8 activations are compared bit-exact.
 * ------------------------------------------------------------------------------------ */
void orc_fwht256(float *v) {
    for (int h = 1; h < ROT; h <<= 1) {
        for (int i = 0; i < ROT; i++) {
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
    for (int j = 0; j < ROT; j++) v[j] = v[j] * 0.0625f;
}

/* Rotate every row of a [R][K] matrix block by block (K % 256 == 0). */
void orc_rotate_rows(const float *in, int64_t R, int64_t K, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        memcpy(out + r * K, in + r * K, (size_t)K * sizeof(float));
        for (int64_t b = 0; b < K; b += ROT) orc_fwht256(out + r * K + b);
    }
}

/* ------------------------------------------------------------------------------------
 * e4m3 group scales.  [card A "Format": weight_s_rel is fp8_e4m3, one per 16 values;
 * "Verification": the file's dtype is F8_E4M3.]  Reading: the OCP E4M3FN encoding
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 * NaN; largest finite 448).  Encoding rounds to nearest with ties to the even code and
 * saturates at 448.
 * ------------------------------------------------------------------------------------ */
double orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)        /* subnormal: m/8 * 2^-6 */
                        : ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* Nearest code by exhaustive search over the 127 non-negative finite codes; on a tie the
 * code with the even mantissa (even code) wins. */
uint8_t orc_e4m3_encode(float x) {
    int neg = signbit(x) ? 1 : 0;
    double a = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(a - orc_e4m3_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* ------------------------------------------------------------------------------------
 * Sampling for the codebook fit.  [card A "Reproducing": the seed pins the codebook
 * fitting, which samples.]  Reading: S = min(N*K, 2^20) values; all of them when
 * N*K <= 2^20, else S positions drawn with replacement, position i being
 * floor(u_i * N*K / 2^64) for u_i the i-th output of SplitMix64 seeded with `seed`
 * (Steele, Lea and Flood 2014; Vigna's 64-bit finaliser constants).
 * ------------------------------------------------------------------------------------ */
uint64_t orc_splitmix64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

int64_t orc_fit_sample(const float *v, int64_t NK, uint64_t seed, float *sample) {
    if (NK <= FIT_SAMPLE_MAX) {
        memcpy(sample, v, (size_t)NK * sizeof(float));
        return NK;
    }
    for (int64_t i = 0; i < FIT_SAMPLE_MAX; i++) {
        uint64_t u = orc_splitmix64_at(seed, (uint64_t)i);
        uint64_t pos = (uint64_t)(((unsigned __int128)u * (unsigned __int128)NK) >> 64);
        sample[i] = v[pos];
    }
    return FIT_SAMPLE_MAX;
}

/* ------------------------------------------------------------------------------------
 * Lloyd-Max codebook fit, per tensor.  [card A "Format": a per-tensor Lloyd-Max codebook
 * of 16 levels fitted to the tensor's own distribution; card B "Model Overview" calls it
 * a 16-level Lloyd-Max codebook.]  Lloyd's alternation, in fp64:
 *   sort the sample ascending (total order, -0 before +0);
 *   start from the mid-quantiles c_j = s[floor((2j+1) S / 32)];
 *   repeat: thresholds t_j = (c_j + c_{j+1}) / 2; cell j = { s : t_{j-1} < s <= t_j };
 *           stop if no cell changed since the previous pass; otherwise every non-empty
 *           cell's level becomes its mean (sum from the running prefix sums of the sorted
 *           sample, divided by the count); an empty cell keeps its level;
 *   at most 100 updates.
 * The running sums P[i] = s[0] + ... + s[i-1] are fp64 in a blocked order (the cards fix no
 * order): the sample is cut into blocks of PREFIX_BLOCK values; within a block the sums run
 * left to right from 0; the block offsets run left to right over the block totals from 0;
 * P[i + 1] = offset of i's block + block-local sum up to i.  One fp64 add per value more
 * than a single left-to-right pass, and every block can be summed at the same time.
 * Returns the number of updates; c16 receives the fp64 levels; bounds17 (nullable) the
 * cell boundaries of the last pass (cell j = sorted indices [b_j, b_{j+1})).
 * ------------------------------------------------------------------------------------ */
#define PREFIX_BLOCK 1024

static int cmp_total(const void *pa, const void *pb) {
    double a = *(const double *)pa, b = *(const double *)pb;
    if (a < b) return -1;
    if (a > b) return 1;
    int sa = signbit(a) ? 1 : 0, sb = signbit(b) ? 1 : 0;
    return sb - sa; /* -0 sorts before +0 */
}

/* number of sorted values <= t */
static int64_t count_le(const double *s, int64_t S, double t) {
    int64_t lo = 0, hi = S;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (s[mid] <= t) lo = mid + 1; else hi = mid;
    }
    return lo;
}

int orc_lloyd_max16(const float *sample, int64_t S, int max_iters, double *c16,
                    int64_t *bounds17) {
    double *s = (double *)malloc((size_t)S * sizeof(double));
    double *P = (double *)malloc((size_t)(S + 1) * sizeof(double));
    for (int64_t i = 0; i < S; i++) s[i] = (double)sample[i];
    qsort(s, (size_t)S, sizeof(double), cmp_total);
    P[0] = 0.0;
    {
        double off = 0.0;
        for (int64_t b0 = 0; b0 < S; b0 += PREFIX_BLOCK) {
            const int64_t b1 = b0 + PREFIX_BLOCK < S ? b0 + PREFIX_BLOCK : S;
            double run = 0.0;
            for (int64_t i = b0; i < b1; i++) {
                run = run + s[i];
                P[i + 1] = off + run;
            }
            off = off + run;
        }
    }

    double c[LEVELS];
    for (int j = 0; j < LEVELS; j++) c[j] = s[((int64_t)(2 * j + 1) * S) / 32];

    int64_t b[LEVELS + 1], prev[LEVELS + 1];
    for (int j = 0; j <= LEVELS; j++) prev[j] = -1;
    int updates = 0;
    for (int pass = 0; pass <= max_iters; pass++) {
        b[0] = 0;
        b[LEVELS] = S;
        for (int j = 0; j < LEVELS - 1; j++) b[j + 1] = count_le(s, S, (c[j] + c[j + 1]) / 2.0);
        int changed = 0;
        for (int j = 0; j <= LEVELS; j++) changed |= (b[j] != prev[j]);
        if (!changed || updates == max_iters) break;
        for (int j = 0; j < LEVELS; j++) {
            int64_t n = b[j + 1] - b[j];
            if (n > 0) c[j] = (P[b[j + 1]] - P[b[j]]) / (double)n;
        }
        memcpy(prev, b, sizeof(b));
        updates++;
    }
    for (int j = 0; j < LEVELS; j++) c16[j] = c[j];
    if (bounds17) memcpy(bounds17, b, sizeof(b));
    free(s);
    free(P);
    return updates;
}

/* ------------------------------------------------------------------------------------
 * Offline weight quantisation.  [card A "Format": a layer is stored as four tensors (4-bit
 * indices packed in bytes, one e4m3 scale per group of 16, one fp32 scale per row, a
 * 16-entry fp32 codebook); the per-tensor codebook, the per-16 e4m3 scale and the per-row
 * fp32 scale each carry one factor of a weight; the rotation comes first.]  Readings:
 *   1. rotate each row in 256-blocks (orc_fwht256);
 *   2. s_ch[r] = max_k |w_rot[r,k]|                                   (row magnitude)
 *   3. s_rel[r,g] = e4m3(gmax[r,g] / s_ch[r]), gmax the group's max |w_rot| (fp32 divide;
 *      0 when s_ch = 0)                                   (group magnitude, relative)
 *   4. v = w_rot / (s_ch * dec(s_rel)) in fp32, using the decoded scale; 0 when the
 *      product is 0;
 *   5. fit the codebook on v (orc_fit_sample, orc_lloyd_max16), cb[j] = (float)c_j;
 *   6. idx = #{ j in 0..14 : (double)v > ((double)cb[j] + (double)cb[j+1]) / 2 }, the
 *      nearest level with ties to the lower index;
 *   7. pack: byte k/2 = idx[k] | idx[k+1] << 4 (element 2j in the low nibble).
 * v_out (nullable) receives the normalised values v [N][K].  Returns the number of
 * Lloyd updates, or -1 if K is not a multiple of 256 [card A "Precision plan": a width
 * that no rotation group divides cannot take the rotation].
 * ------------------------------------------------------------------------------------ */
int orc_quantize_weight(const float *W, int64_t N, int64_t K, uint64_t seed, int8_t *packed,
                        uint8_t *s_rel, float *s_ch, float *cb, float *v_out) {
    if (N <= 0 || K <= 0 || K % ROT != 0) return -1;
    const int64_t G = K / GRP;
    float *v = (float *)malloc((size_t)(N * K) * sizeof(float));
    orc_rotate_rows(W, N, K, v); /* v holds w_rot for now */

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; r++) {
        float *row = v + r * K;
        float rmax = 0.0f;
        for (int64_t k = 0; k < K; k++) rmax = fmaxf(rmax, fabsf(row[k]));
        s_ch[r] = rmax;
        for (int64_t g = 0; g < G; g++) {
            float gmax = 0.0f;
            for (int i = 0; i < GRP; i++) gmax = fmaxf(gmax, fabsf(row[g * GRP + i]));
            uint8_t code = (rmax > 0.0f) ? orc_e4m3_encode(gmax / rmax) : 0;
            s_rel[r * G + g] = code;
            float d = rmax * (float)orc_e4m3_decode(code);
            for (int i = 0; i < GRP; i++) {
                float w = row[g * GRP + i];
                row[g * GRP + i] = (d > 0.0f) ? w / d : 0.0f;
            }
        }
    }

    int64_t NK = N * K;
    int64_t smax = NK < FIT_SAMPLE_MAX ? NK : FIT_SAMPLE_MAX;
    float *sample = (float *)malloc((size_t)smax * sizeof(float));
    int64_t S = orc_fit_sample(v, NK, seed, sample);
    double c[LEVELS];
    int updates = orc_lloyd_max16(sample, S, FIT_MAX_ITERS, c, NULL);
    for (int j = 0; j < LEVELS; j++) cb[j] = (float)c[j];
    free(sample);

    double mid[LEVELS - 1];
    for (int j = 0; j < LEVELS - 1; j++) mid[j] = ((double)cb[j] + (double)cb[j + 1]) / 2.0;

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; r++) {
        for (int64_t k = 0; k < K; k += 2) {
            int idx[2];
            for (int t = 0; t < 2; t++) {
                double x = (double)v[r * K + k + t];
                int n = 0;
                for (int j = 0; j < LEVELS - 1; j++) n += (x > mid[j]) ? 1 : 0;
                idx[t] = n;
            }
            packed[r * (K / 2) + k / 2] = (int8_t)(uint8_t)(idx[0] | (idx[1] << 4));
        }
    }
    if (v_out) memcpy(v_out, v, (size_t)NK * sizeof(float));
    free(v);
    return updates;
}

/* ------------------------------------------------------------------------------------
 * Activation preparation.  [card B "Model Overview": 4-bit weights with int8
 * activations; card A "Format": executed on int8 GEMM.]  Readings: the activations take
 * the same 256-block rotation as the weights' in_features (so the rotated product equals
 * the unrotated one, the rotation being orthonormal and symmetric); then per token
 * (row) symmetric int8: amax = max |x_rot|, s_x = amax / 127 (fp32 divide),
 * x_q = clamp(rint(x_rot / s_x), -127, 127) with IEEE divide and ties to even; a row with
 * amax = 0 gets s_x = 0 and x_q = 0.  Input is fp32 (bf16 input is widened exactly by the
 * caller).
 * ------------------------------------------------------------------------------------ */
void orc_prepare(const float *x, int64_t M, int64_t K, int8_t *xq, float *sx) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float *t = (float *)malloc((size_t)K * sizeof(float));
        memcpy(t, x + m * K, (size_t)K * sizeof(float));
        for (int64_t b = 0; b < K; b += ROT) orc_fwht256(t + b);
        float amax = 0.0f;
        for (int64_t k = 0; k < K; k++) amax = fmaxf(amax, fabsf(t[k]));
        float s = amax / 127.0f;
        sx[m] = s;
        for (int64_t k = 0; k < K; k++) {
            int q = 0;
            if (amax > 0.0f) {
                float r = rintf(t[k] / s);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q = (int)r;
            }
            xq[m * K + k] = (int8_t)q;
        }
        free(t);
    }
}

/* ------------------------------------------------------------------------------------
 * Dequantised weight, exact in fp64: w_hat[r,k] = s_ch[r] * dec(s_rel[r,k/16]) *
 * cb[idx[r,k]] (24 + 4 + 24 significant bits fit in 53).  [card A "Format": a weight is
 * the product of its codebook level, its group's e4m3 scale and its row's fp32 scale.]
 * ------------------------------------------------------------------------------------ */
static inline int unpack_idx(const int8_t *packed_row, int64_t k) {
    uint8_t byte = (uint8_t)packed_row[k / 2];
    return (k % 2 == 0) ? (byte & 15) : (byte >> 4);
}

void orc_dequant(const int8_t *packed, const uint8_t *s_rel, const float *s_ch, const float *cb,
                 int64_t N, int64_t K, double *w_hat) {
    const int64_t G = K / GRP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; r++) {
        for (int64_t k = 0; k < K; k++) {
            int j = unpack_idx(packed + r * (K / 2), k);
            w_hat[r * K + k] =
                (double)s_ch[r] * orc_e4m3_decode(s_rel[r * G + k / GRP]) * (double)cb[j];
        }
    }
}

/* ------------------------------------------------------------------------------------
 * The product.  [card A "Why this exists" / "Format": the layer runs on the int8 GEMM
 * path with a codebook dequantisation step on top.]  Definition:
 *   y[m,r] = sum_k (s_x[m] * x_q[m,k]) * w_hat[r,k]
 * accumulated in fp64 in natural k order, with A[m,r] = sum_k |(s_x x_q)[m,k] w_hat[r,k]|
 * the scale against which the floating-point tolerance is stated.  rows / toks (nullable)
 * select a subset: outputs are [ntok][nrow].
 * ------------------------------------------------------------------------------------ */
void orc_linear_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K, const int8_t *packed,
                    const uint8_t *s_rel, const float *s_ch, const float *cb, int64_t N,
                    const int64_t *rows, int64_t nrow, const int64_t *toks, int64_t ntok,
                    double *y, double *A) {
    if (!rows) nrow = N;
    if (!toks) ntok = M;
    const int64_t G = K / GRP;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrow; ri++) {
        int64_t r = rows ? rows[ri] : ri;
        double *w = (double *)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; k++) {
            int j = unpack_idx(packed + r * (K / 2), k);
            w[k] = (double)s_ch[r] * orc_e4m3_decode(s_rel[r * G + k / GRP]) * (double)cb[j];
        }
        for (int64_t ti = 0; ti < ntok; ti++) {
            int64_t m = toks ? toks[ti] : ti;
            double acc = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double t = ((double)sx[m] * (double)xq[m * K + k]) * w[k];
                acc += t;
                a += fabs(t);
            }
            y[ti * nrow + ri] = acc;
            A[ti * nrow + ri] = a;
        }
        free(w);
    }
}

/* ------------------------------------------------------------------------------------
 * The int8 execution of the codebook product.  [card A "Why this exists": the W4A8 layer
 * executes on the same int8 GEMM path as INT8 and adds a codebook dequantisation step.]
 * Reading: the fp32 codebook is carried on the int8 path as
 *   s_cb = max_j |cb[j]| / 127 (fp32),  cb_i8[j] = rint(cb[j] / s_cb) (fp32, ties even),
 * the per-16 group partial P[m,r,g] = sum_{k in g} x_q[m,k] * cb_i8[idx[r,k]] is an exact
 * integer, and
 *   y8[m,r] = s_x[m] * s_ch[r] * s_cb * sum_g dec(s_rel[r,g]) * P[m,r,g]      (fp64)
 * with A8 the same sum of absolute products.  scb_out / cbi8_out (nullable) receive s_cb
 * and cb_i8; P (nullable) receives the partials [ntok][nrow][G].
 * ------------------------------------------------------------------------------------ */
void orc_codebook_i8(const float *cb, float *scb_out, int8_t *cbi8_out) {
    float mx = 0.0f;
    for (int j = 0; j < LEVELS; j++) mx = fmaxf(mx, fabsf(cb[j]));
    float s = mx / 127.0f;
    for (int j = 0; j < LEVELS; j++) cbi8_out[j] = (int8_t)((s > 0.0f) ? (int)rintf(cb[j] / s) : 0);
    *scb_out = s;
}

void orc_linear_i8_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K,
                       const int8_t *packed, const uint8_t *s_rel, const float *s_ch,
                       const float *cb, int64_t N, const int64_t *rows, int64_t nrow,
                       const int64_t *toks, int64_t ntok, double *y8, double *A8, int32_t *P) {
    if (!rows) nrow = N;
    if (!toks) ntok = M;
    const int64_t G = K / GRP;
    float s_cb;
    int8_t cbi8[LEVELS];
    orc_codebook_i8(cb, &s_cb, cbi8);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrow; ri++) {
        int64_t r = rows ? rows[ri] : ri;
        for (int64_t ti = 0; ti < ntok; ti++) {
            int64_t m = toks ? toks[ti] : ti;
            double acc = 0.0, a = 0.0;
            for (int64_t g = 0; g < G; g++) {
                int32_t p = 0;
                double pabs = 0.0;
                for (int i = 0; i < GRP; i++) {
                    int64_t k = g * GRP + i;
                    int32_t prod = (int32_t)xq[m * K + k] * (int32_t)cbi8[unpack_idx(packed + r * (K / 2), k)];
                    p += prod;
                    pabs += fabs((double)prod);
                }
                double sg = orc_e4m3_decode(s_rel[r * G + g]);
                acc += sg * (double)p;
                a += fabs(sg) * pabs;
                if (P) P[(ti * nrow + ri) * G + g] = p;
            }
            double scale = (double)sx[m] * (double)s_ch[r] * (double)s_cb;
            y8[ti * nrow + ri] = scale * acc;
            A8[ti * nrow + ri] = fabs(scale) * a;
        }
    }
}

/* ------------------------------------------------------------------------------------
 * Requantised int8 weights: the second reading of the int8 execution.  [card A "Why this
 * exists": the W4A8 layer runs on the same int8 GEMM path as INT8 with a codebook
 * dequantisation step added.]  Where orc_linear_i8_ref keeps the group scale outside the
 * integer sum (one fold per 16 values), this reading decodes each weight with its group
 * scale and rounds it to int8 on one per-tensor step, so a single integer sum covers the
 * whole row and the scales enter once:
 *   s_cb     = max_j |cb[j]| / 127                                   (fp32, as orc_codebook_i8)
 *   t[c][j]  = rint(fl(dec(c) * cb[j]) / s_cb)  for each e4m3 code c   (fp32 product, then fp32
 *              quotient, ties to even; clamped to [-127, 127]; 0 where the quotient is NaN)
 *   q[r,k]   = t[s_rel[r,k/16]][idx[r,k]]
 *   acc[m,r] = sum_k x_q[m,k] q[r,k]                                 (exact integer)
 *   y[m,r]   = fl(fl(fl(acc) * fl(s_ch[r] * s_cb)) * s_x[m])          (fp32, in this order)
 * No value is clamped when every |dec(s_rel)| <= 1, which orc_quantize_weight guarantees
 * (the group that holds a row's largest magnitude has relative scale 1).  The rounding
 * step is s_cb in units of s_ch[r], so |q s_cb - dec cb| <= s_cb / 2 for each weight.
 * ------------------------------------------------------------------------------------ */
void orc_rq_table(const float *cb, int8_t *tab /* [256][16] */) {
    float mx = 0.0f;
    for (int j = 0; j < LEVELS; j++) mx = fmaxf(mx, fabsf(cb[j]));
    const float s = mx / 127.0f;
    for (int c = 0; c < 256; c++) {
        const float d = (float)orc_e4m3_decode((uint8_t)c);
        for (int j = 0; j < LEVELS; j++) {
            const float prod = d * cb[j];
            const float v = prod / s;
            float qv = 0.0f;
            if (!isnan(v)) {
                qv = rintf(v);
                qv = qv > 127.0f ? 127.0f : (qv < -127.0f ? -127.0f : qv);
            }
            tab[c * LEVELS + j] = (int8_t)qv;
        }
    }
}

void orc_linear_rq_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K,
                       const int8_t *packed, const uint8_t *s_rel, const float *s_ch,
                       const float *cb, int64_t N, const int64_t *rows, int64_t nrow,
                       const int64_t *toks, int64_t ntok, float *y) {
    if (!rows) nrow = N;
    if (!toks) ntok = M;
    const int64_t G = K / GRP;
    int8_t tab[256 * LEVELS];
    orc_rq_table(cb, tab);
    float mx = 0.0f;
    for (int j = 0; j < LEVELS; j++) mx = fmaxf(mx, fabsf(cb[j]));
    const float s_cb = mx / 127.0f;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrow; ri++) {
        int64_t r = rows ? rows[ri] : ri;
        int8_t *q = (int8_t *)malloc((size_t)K);
        for (int64_t k = 0; k < K; k++)
            q[k] = tab[s_rel[r * G + k / GRP] * LEVELS + unpack_idx(packed + r * (K / 2), k)];
        const float sw = s_ch[r] * s_cb;
        for (int64_t ti = 0; ti < ntok; ti++) {
            int64_t m = toks ? toks[ti] : ti;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; k++) acc += (int64_t)xq[m * K + k] * (int64_t)q[k];
            const float t = (float)acc * sw;
            y[ti * nrow + ri] = t * sx[m];
        }
        free(q);
    }
}

/* ---------------------------------------------------------------- W8A8 comparator
 * The INT8 ConvRot format the W4A8 layer is weighed against [card A, "Why this exists": an
 * INT8 ConvRot build of the same model, about twice the weight bytes].  The cards give no
 * more detail; the reading taken is the plainest one next to the per-token int8
 * activations: each weight row takes the same 256-block rotation, then one fp32 scale per row
 * s_w = max |w_rot| / 127 and codes w_q = clamp(rint(w_rot / s_w), -127, 127) (IEEE
 * division, ties to even); a zero row gives s_w = 0 and w_q = 0.  No codebook, no groups. */
void orc_quantize_w8(const float *W, int64_t N, int64_t K, int8_t *wq, float *sw) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; r++) {
        float *t = (float *)malloc((size_t)K * sizeof(float));
        memcpy(t, W + r * K, (size_t)K * sizeof(float));
        for (int64_t b = 0; b < K; b += ROT) orc_fwht256(t + b);
        float rmax = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float a = fabsf(t[k]);
            if (a > rmax) rmax = a;
        }
        const float s = rmax / 127.0f;
        sw[r] = s;
        for (int64_t k = 0; k < K; k++) {
            float q = 0.0f;
            if (rmax > 0.0f) {
                q = rintf(t[k] / s);
                q = q > 127.0f ? 127.0f : (q < -127.0f ? -127.0f : q);
            }
            wq[r * K + k] = (int8_t)q;
        }
        free(t);
    }
}

/* y[m][r] = s_x[m] s_w[r] sum_k x_q[m][k] w_q[r][k] in fp64; the integer sum is exact. */
void orc_linear_w8_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K, const int8_t *wq,
                       const float *sw, int64_t N, double *y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; r++) {
        for (int64_t m = 0; m < M; m++) {
            int64_t dot = 0;
            for (int64_t k = 0; k < K; k++) dot += (int64_t)xq[m * K + k] * (int64_t)wq[r * K + k];
            y[m * N + r] = (double)sx[m] * (double)sw[r] * (double)dot;
        }
    }
}
