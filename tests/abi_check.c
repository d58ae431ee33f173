/*
 * The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure only; tests/test_sanitize.py builds the library's api.hip with host-side
 * sanitizers, links it with the other objects and runs this driver, no GPU needed).  Every
 * C-ABI entry point is called with invalid arguments -- null, misaligned and out-of-range --
 * and must return its documented status before touching the GPU; the metadata calls run in
 * full.  A sanitizer report aborts the run.  Prints "ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "w4a8.h"

#define FAKE ((void *)(uintptr_t)0x10000) /* 16-byte aligned, never dereferenced */
#define MIS ((void *)(uintptr_t)0x10008)  /* misaligned */

static int failures = 0;
#define EXPECT(call, want)                                                                     \
    do {                                                                                       \
        const int got_ = (int)(call);                                                          \
        if (got_ != (want)) {                                                                  \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_,   \
                    (int)(want));                                                              \
            failures++;                                                                        \
        }                                                                                      \
    } while (0)

static int lin(const void *xq, const void *sx, int64_t M, int64_t K, const void *pk, const void *sr,
               const void *sc, const void *cb, int64_t N, void *y, int ydt, int algo) {
    return w4a8_linear_algo(xq, sx, M, K, pk, sr, sc, cb, N, y, ydt, algo, NULL);
}

int main(void) {
    /* metadata */
    EXPECT(w4a8_version(), 100);
    for (int s = -1; s < 10; s++) {
        const char *t = w4a8_status_string(s);
        if (!t || !t[0]) failures++;
    }
    EXPECT(w4a8_quantize_weight_workspace(17408, 5120) == 12583168, 1);
    EXPECT(w4a8_quantize_weight_workspace(0, 512), 0);
    EXPECT(w4a8_quantize_weight_workspace(4, 4304), 0);
    EXPECT(w4a8_quantize_weight_workspace(-1, 256), 0);
    EXPECT(w4a8_quantize_weight_workspace((int64_t)1 << 40, 256), 0);
    EXPECT(w4a8_linear_pick(1, 1, 4304), -W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_pick(0, 1, 512), -W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_pick(INT64_MAX, INT64_MAX, 256) > 0, 1);

    /* linear */
    EXPECT(lin(NULL, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, 0), W4A8_ERR_NULL);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, NULL, 256, FAKE, 0, 0), W4A8_ERR_NULL);
    EXPECT(lin(FAKE, FAKE, 0, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, 0), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 4, 300, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, 0), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, -3, 512, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, 0), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, INT64_MAX, 512, FAKE, FAKE, FAKE, FAKE, INT64_MAX, FAKE, 0, 0), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 4, INT64_MAX - 255, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, 0), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 7, 0), W4A8_ERR_DTYPE);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, 9), W4A8_ERR_DTYPE);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, -1), W4A8_ERR_DTYPE);
    EXPECT(lin(MIS, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, 0), W4A8_ERR_ALIGN);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, MIS, 0, 0), W4A8_ERR_ALIGN);
    EXPECT(lin(FAKE, FAKE, 8, 5120, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, W4A8_ALGO_GEMV), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 65, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, W4A8_ALGO_MFMA_SKINNY), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 4, 131328, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, W4A8_ALGO_MFMA_RQ), W4A8_ERR_SHAPE);
    const int64_t huge = ((int64_t)1 << 31) - 1;
    EXPECT(lin(FAKE, FAKE, huge, 512, FAKE, FAKE, FAKE, FAKE, huge, FAKE, 0, W4A8_ALGO_MFMA_I8), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, huge, 512, FAKE, FAKE, FAKE, FAKE, huge, FAKE, 0, W4A8_ALGO_MFMA_F16), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, huge, 512, FAKE, FAKE, FAKE, FAKE, huge, FAKE, 0, W4A8_ALGO_MFMA_RQ), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, huge, 512, FAKE, FAKE, FAKE, FAKE, huge, FAKE, 0, W4A8_ALGO_MFMA_I8_FOLD), W4A8_ERR_SHAPE);
    EXPECT(lin(FAKE, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, 7), W4A8_ERR_DTYPE);
    EXPECT(w4a8_linear(NULL, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, NULL), W4A8_ERR_NULL);

    /* prepare, quantize (both forms) */
    EXPECT(w4a8_prepare_activation(NULL, 0, 4, 512, FAKE, FAKE, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_prepare_activation(FAKE, 0, 4, 300, FAKE, FAKE, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_prepare_activation(FAKE, 0, INT64_MAX, 512, FAKE, FAKE, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_prepare_activation(FAKE, 5, 4, 512, FAKE, FAKE, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_prepare_activation(MIS, 0, 4, 512, FAKE, FAKE, NULL), W4A8_ERR_ALIGN);
    const size_t need = w4a8_quantize_weight_workspace(8, 256);
    EXPECT(w4a8_quantize_weight(NULL, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_quantize_weight(FAKE, 0, 8, 4304, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_quantize_weight(FAKE, 2, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_quantize_weight(FAKE, 0, 8, 256, 0, MIS, FAKE, FAKE, FAKE, FAKE, need, NULL), W4A8_ERR_ALIGN);
    EXPECT(w4a8_quantize_weight(FAKE, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, NULL), W4A8_ERR_WORKSPACE);
    EXPECT(w4a8_quantize_weight(FAKE, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, NULL, need, NULL), W4A8_ERR_WORKSPACE);
    EXPECT(w4a8_quantize_weight_noalloc(NULL, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_quantize_weight_noalloc(FAKE, 0, 8, 300, 0, FAKE, FAKE, FAKE, FAKE, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_quantize_weight_noalloc(FAKE, 3, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_quantize_weight_noalloc(FAKE, 0, 8, 256, 0, FAKE, MIS, FAKE, FAKE, NULL), W4A8_ERR_ALIGN);

    /* forward */
    EXPECT(w4a8_forward(NULL, 0, 1, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, FAKE, FAKE, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_forward(FAKE, 0, 1, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, NULL, FAKE, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_forward(FAKE, 0, 1, 4304, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, FAKE, FAKE, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_forward(FAKE, 4, 1, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, FAKE, FAKE, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_forward(MIS, 0, 1, 512, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 0, FAKE, FAKE, NULL), W4A8_ERR_ALIGN);

    /* several layers */
    w4a8_layer t[9];
    for (int g = 0; g < 9; g++) {
        t[g].packed = FAKE; t[g].s_rel = FAKE; t[g].s_channel = FAKE; t[g].codebook = FAKE;
        t[g].N = 256; t[g].y = FAKE;
    }
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 2, NULL, 0, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 0, t, 0, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 9, t, 0, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 300, 2, t, 0, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 2, t, 5, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_linear_multi(NULL, FAKE, 1, 512, 2, t, 0, NULL), W4A8_ERR_NULL);
    t[1].packed = NULL;
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 2, t, 0, NULL), W4A8_ERR_NULL);
    t[1].packed = FAKE;
    t[0].y = MIS;
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 2, t, 0, NULL), W4A8_ERR_ALIGN);
    t[0].y = FAKE;
    t[0].N = 0;
    EXPECT(w4a8_linear_multi(FAKE, FAKE, 1, 512, 2, t, 0, NULL), W4A8_ERR_SHAPE);
    t[0].N = 256;
    EXPECT(w4a8_forward_multi(NULL, 0, 1, 512, 2, t, 0, FAKE, FAKE, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_forward_multi(FAKE, 4, 1, 512, 2, t, 0, FAKE, FAKE, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_forward_multi(MIS, 0, 1, 512, 2, t, 0, FAKE, FAKE, NULL), W4A8_ERR_ALIGN);
    EXPECT(w4a8_forward_multi(FAKE, 0, 1, 512, 2, t, 0, NULL, FAKE, NULL), W4A8_ERR_NULL);

    /* the product with a workspace (checks that return before any device call) */
    EXPECT(w4a8_linear_workspace_bytes(8, 256, 300), -W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_workspace_bytes(0, 256, 512), -W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_workspace_bytes(1, 17408, 5120), 0);     /* the GEMV: no workspace */
    EXPECT(w4a8_linear_workspace_bytes(2048, 5120, 17408), 0);  /* prefill: no workspace */
    EXPECT(w4a8_linear_ws(NULL, FAKE, 32, 8192, FAKE, FAKE, FAKE, FAKE, 5120, FAKE, 0, FAKE, 1 << 20, NULL),
           W4A8_ERR_NULL);
    EXPECT(w4a8_linear_ws(FAKE, FAKE, 32, 8200, FAKE, FAKE, FAKE, FAKE, 5120, FAKE, 0, FAKE, 1 << 20, NULL),
           W4A8_ERR_SHAPE);
    EXPECT(w4a8_linear_ws(FAKE, FAKE, 32, 8192, FAKE, FAKE, FAKE, FAKE, 5120, FAKE, 7, FAKE, 1 << 20, NULL),
           W4A8_ERR_DTYPE);
    EXPECT(w4a8_linear_ws(FAKE, FAKE, 32, 8192, FAKE, FAKE, FAKE, FAKE, 5120, FAKE, 0, MIS, 1 << 20, NULL),
           W4A8_ERR_ALIGN);

    /* the W8A8 comparator */
    EXPECT(w4a8_w8a8_quantize_weight(NULL, 0, 8, 256, FAKE, FAKE, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_w8a8_quantize_weight(FAKE, 0, 8, 131072 + 256, FAKE, FAKE, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_w8a8_quantize_weight(FAKE, 2, 8, 256, FAKE, FAKE, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_w8a8_quantize_weight(FAKE, 0, 8, 256, MIS, FAKE, NULL), W4A8_ERR_ALIGN);
    EXPECT(w4a8_w8a8_linear(NULL, FAKE, 4, 512, FAKE, FAKE, 256, FAKE, 0, 0, NULL), W4A8_ERR_NULL);
    EXPECT(w4a8_w8a8_linear(FAKE, FAKE, 4, 300, FAKE, FAKE, 256, FAKE, 0, 0, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_w8a8_linear(FAKE, FAKE, 4, 512, FAKE, FAKE, 256, FAKE, 2, 0, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_w8a8_linear(FAKE, FAKE, 4, 512, FAKE, FAKE, 256, FAKE, 0, W4A8_ALGO_MFMA_F16, NULL), W4A8_ERR_DTYPE);
    EXPECT(w4a8_w8a8_linear(FAKE, FAKE, 5, 512, FAKE, FAKE, 256, FAKE, 0, W4A8_ALGO_GEMV, NULL), W4A8_ERR_SHAPE);
    EXPECT(w4a8_w8a8_linear(FAKE, MIS, 4, 512, FAKE, FAKE, 256, FAKE, 0, 0, NULL), W4A8_ERR_ALIGN);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
