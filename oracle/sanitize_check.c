/*
 * Memory and undefined-behaviour check of the CPU oracle (test infrastructure only): every
 * oracle entry point runs on small, ragged and edge-case inputs in a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py compiles it with
 * w4a8_oracle.c and runs it).  Any out-of-bounds access, leak, signed overflow, misaligned or
 * invalid shift aborts the run; a few identities are checked on the way so that the calls do
 * real work.  Exit status 0 and a final "ok" line on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_num_threads(void);
void orc_fwht256(float *v);
void orc_rotate_rows(const float *in, int64_t R, int64_t K, float *out);
double orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(float x);
uint64_t orc_splitmix64_at(uint64_t seed, uint64_t i);
int64_t orc_fit_sample(const float *v, int64_t NK, uint64_t seed, float *sample);
int orc_lloyd_max16(const float *sample, int64_t S, int max_iters, double *c16, int64_t *bounds17);
int orc_quantize_weight(const float *W, int64_t N, int64_t K, uint64_t seed, int8_t *packed,
                        uint8_t *s_rel, float *s_ch, float *cb, float *v_out);
void orc_prepare(const float *x, int64_t M, int64_t K, int8_t *xq, float *sx);
void orc_dequant(const int8_t *packed, const uint8_t *s_rel, const float *s_ch, const float *cb,
                 int64_t N, int64_t K, double *w_hat);
void orc_linear_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K, const int8_t *packed,
                    const uint8_t *s_rel, const float *s_ch, const float *cb, int64_t N,
                    const int64_t *rows, int64_t nrow, const int64_t *toks, int64_t ntok,
                    double *y, double *A);
void orc_codebook_i8(const float *cb, float *scb_out, int8_t *cbi8_out);
void orc_linear_i8_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K,
                       const int8_t *packed, const uint8_t *s_rel, const float *s_ch,
                       const float *cb, int64_t N, const int64_t *rows, int64_t nrow,
                       const int64_t *toks, int64_t ntok, double *y8, double *A8, int32_t *P);
void orc_rq_table(const float *cb, int8_t *tab);
void orc_linear_rq_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K,
                       const int8_t *packed, const uint8_t *s_rel, const float *s_ch,
                       const float *cb, int64_t N, const int64_t *rows, int64_t nrow,
                       const int64_t *toks, int64_t ntok, float *y);
void orc_quantize_w8(const float *W, int64_t N, int64_t K, int8_t *wq, float *sw);
void orc_linear_w8_ref(const int8_t *xq, const float *sx, int64_t M, int64_t K, const int8_t *wq,
                       const float *sw, int64_t N, double *y);

static uint64_t g_state = 12345;
static double uniform(void) { /* xorshift64*, in [0, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 2685821657736338717ULL) >> 11) * 0x1.0p-53;
}
static float *randn(int64_t n, float scale) {
    float *a = malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; i++) {
        const double u1 = uniform() + 1e-300, u2 = uniform();
        a[i] = (float)(scale * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
    }
    return a;
}
static void check(int ok, const char *what) {
    if (!ok) {
        fprintf(stderr, "check failed: %s\n", what);
        exit(1);
    }
}

/* one layer: quantise, then every product route on it */
static void layer_case(int64_t N, int64_t K, int64_t M, uint64_t seed) {
    float *W = randn(N * K, 0.02f);
    if (N > 2) memset(W + K, 0, (size_t)K * sizeof(float));             /* a zero row */
    int8_t *packed = malloc((size_t)(N * K / 2));
    uint8_t *s_rel = malloc((size_t)(N * K / 16));
    float *s_ch = malloc((size_t)N * sizeof(float)), cb[16];
    float *v = malloc((size_t)(N * K) * sizeof(float));
    check(orc_quantize_weight(W, N, K, seed, packed, s_rel, s_ch, cb, v) >= 0, "quantize_weight");
    for (int j = 1; j < 16; j++) check(cb[j - 1] <= cb[j], "codebook ascending");

    float *x = randn(M * K, 1.0f);
    if (M > 1) memset(x + K, 0, (size_t)K * sizeof(float));              /* a zero token */
    int8_t *xq = malloc((size_t)(M * K));
    float *sx = malloc((size_t)M * sizeof(float));
    orc_prepare(x, M, K, xq, sx);
    if (M > 1) check(sx[1] == 0.0f, "zero token scale");

    double *w_hat = malloc((size_t)(N * K) * sizeof(double));
    orc_dequant(packed, s_rel, s_ch, cb, N, K, w_hat);

    double *y = malloc((size_t)(M * N) * sizeof(double)), *A = malloc((size_t)(M * N) * sizeof(double));
    orc_linear_ref(xq, sx, M, K, packed, s_rel, s_ch, cb, N, NULL, N, NULL, M, y, A);
    for (int64_t i = 0; i < M * N; i++) check(fabs(y[i]) <= A[i] * (1 + 1e-12), "|y| <= A");
    /* the dense route: y = s_x * sum x_q * w_hat */
    for (int64_t m = 0; m < M; m++)
        for (int64_t r = 0; r < N; r++) {
            double d = 0.0;
            for (int64_t k = 0; k < K; k++) d += (double)xq[m * K + k] * w_hat[r * K + k];
            d *= sx[m];
            check(fabs(d - y[m * N + r]) <= 1e-9 * (A[m * N + r] + 1e-300), "dense route");
        }

    /* subsets of rows and tokens (last and first), int8-codebook and requantised routes */
    int64_t rows[2] = {N - 1, 0}, toks[2] = {M - 1, 0};
    const int64_t nr = N > 1 ? 2 : 1, nt = M > 1 ? 2 : 1;
    double ys[4], As[4], y8[4], A8[4];
    int32_t *P = malloc((size_t)(nr * nt * (K / 16)) * sizeof(int32_t));
    orc_linear_ref(xq, sx, M, K, packed, s_rel, s_ch, cb, N, rows, nr, toks, nt, ys, As);
    check(ys[0] == y[(M - 1) * N + (N - 1)], "subset matches full");
    orc_linear_i8_ref(xq, sx, M, K, packed, s_rel, s_ch, cb, N, rows, nr, toks, nt, y8, A8, P);
    double *y8f = malloc((size_t)(M * N) * sizeof(double)), *A8f = malloc((size_t)(M * N) * sizeof(double));
    orc_linear_i8_ref(xq, sx, M, K, packed, s_rel, s_ch, cb, N, NULL, N, NULL, M, y8f, A8f, NULL);
    check(y8f[(M - 1) * N + (N - 1)] == y8[0], "i8 subset matches full");
    float scb;
    int8_t cbi8[16], tab[256 * 16];
    orc_codebook_i8(cb, &scb, cbi8);
    orc_rq_table(cb, tab);
    float *yq = malloc((size_t)(M * N) * sizeof(float)), yqs[4];
    orc_linear_rq_ref(xq, sx, M, K, packed, s_rel, s_ch, cb, N, NULL, N, NULL, M, yq);
    orc_linear_rq_ref(xq, sx, M, K, packed, s_rel, s_ch, cb, N, rows, nr, toks, nt, yqs);
    check(yqs[0] == yq[(M - 1) * N + (N - 1)], "rq subset matches full");

    int8_t *wq = malloc((size_t)(N * K));
    float *sw = malloc((size_t)N * sizeof(float));
    orc_quantize_w8(W, N, K, wq, sw);
    double *yw = malloc((size_t)(M * N) * sizeof(double));
    orc_linear_w8_ref(xq, sx, M, K, wq, sw, N, yw);

    free(W); free(packed); free(s_rel); free(s_ch); free(v); free(x); free(xq); free(sx);
    free(w_hat); free(y); free(A); free(P); free(yq); free(wq); free(sw); free(yw); free(y8f); free(A8f);
}

int main(void) {
    check(orc_num_threads() >= 1, "threads");

    /* rotation: self-inverse, and the row version agrees with the block version */
    float *a = randn(256, 1.0f), b[256];
    memcpy(b, a, sizeof(b));
    orc_fwht256(b);
    orc_fwht256(b);
    for (int i = 0; i < 256; i++) check(fabsf(a[i] - b[i]) <= 1e-5f * (1.0f + fabsf(a[i])), "fwht self-inverse");
    float *rows_in = randn(3 * 512, 1.0f), *rows_out = malloc(3 * 512 * sizeof(float));
    orc_rotate_rows(rows_in, 3, 512, rows_out);
    memcpy(b, rows_in + 512 + 256, sizeof(b));
    orc_fwht256(b);
    check(memcmp(b, rows_out + 512 + 256, sizeof(b)) == 0, "rotate_rows block");
    free(a); free(rows_in); free(rows_out);

    /* e4m3: every code, and the encoder over a sweep (round trip on finite codes) */
    for (int c = 0; c < 256; c++) {
        const double d = orc_e4m3_decode((uint8_t)c);
        if (!isnan(d) && c != 0x80) check(orc_e4m3_encode((float)d) == c, "e4m3 round trip");
    }
    for (int i = -2000; i <= 2000; i++) (void)orc_e4m3_encode((float)ldexp(i, -6));
    (void)orc_e4m3_encode(1e30f);
    (void)orc_e4m3_encode(-1e-30f);
    (void)orc_splitmix64_at(0, 0);
    (void)orc_splitmix64_at(~0ULL, ~0ULL);

    /* fit sample: all values, and a strided sample of a larger set */
    const int64_t big = (1 << 20) + 37;
    float *vals = randn(big, 1.0f), *sample = malloc((size_t)big * sizeof(float));
    check(orc_fit_sample(vals, 1000, 0, sample) == 1000, "sample small");
    const int64_t S = orc_fit_sample(vals, big, 7, sample);
    check(S == (1 << 20), "sample size");
    double c16[16];
    int64_t bounds[17];
    check(orc_lloyd_max16(sample, 5000, 100, c16, bounds) >= 0, "lloyd");
    check(orc_lloyd_max16(sample, 17, 100, c16, bounds) >= 0, "lloyd tiny");
    free(vals); free(sample);

    /* layers: one block, ragged rows and tokens, a longer row */
    layer_case(1, 256, 1, 0);
    layer_case(5, 512, 3, 1);
    layer_case(17, 768, 4, 2);
    layer_case(3, 4096, 2, 3);
    printf("ok\n");
    return 0;
}
