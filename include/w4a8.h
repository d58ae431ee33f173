/*
 * w4a8.h -- C ABI of the MI355X (gfx950) W4A8 codebook linear layer library (libw4a8.so).
 *
 * The layer is the asym_w4a8_int8 ("ConvRot") quantised linear described by the model
 * cards "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI" (sections "Format", "Why this
 * exists", "Reproducing") and "Qwen3.8-27B-W4A8 (for ComfyUI)" (section "Model
 * Overview").  One quantised layer of N output rows and K input features is four tensors:
 *
 *   packed     int8   [N][K/2]   4-bit codebook indices, two per byte; element 2j of a row
 *                                sits in the low nibble of byte j, element 2j+1 in the high
 *   s_rel      uint8  [N][K/16]  group scales, OCP fp8 E4M3FN bit patterns, one per 16 values
 *   s_channel  fp32   [N]        per-output-row scale
 *   codebook   fp32   [16]       the tensor's 16 levels (a Lloyd-Max fit; any 16 values work)
 *
 * and the layer computes, with activations rotated and quantised per token,
 *
 *   y[m][r] = s_x[m] * sum_k x_q[m][k] * s_channel[r] * dec(s_rel[r][k/16]) * codebook[idx[r][k]]
 *
 * where the rotation is the orthonormal Sylvester Hadamard transform of order 256 applied
 * to every 256-block of the K axis of both weights (offline) and activations (per call).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, row-major and
 *    contiguous, owned by the caller, and at least 16-byte aligned.  The library keeps no
 *    reference to them after the call returns and allocates no device memory.
 *  - `stream` is a hipStream_t (0 = the null stream).  Work is enqueued asynchronously
 *    on it; the call returns as soon as the work is enqueued.
 *  - Arguments are validated before anything is enqueued: on a non-zero status nothing
 *    was launched and no output was touched.  Faults inside kernels are asynchronous and
 *    surface at the caller's next synchronisation on the stream.
 *  - Non-finite inputs are outside the contract (no fault; unspecified output).
 *  - Calls on distinct streams may run concurrently; calls are re-entrant and thread-safe.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define W4A8_API __attribute__((visibility("default")))
#else
#define W4A8_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A8_OK = 0,
    W4A8_ERR_NULL = 1,       /* a required pointer is NULL */
    W4A8_ERR_SHAPE = 2,      /* M, N or K out of range; K not a multiple of 256 */
    W4A8_ERR_DTYPE = 3,      /* unknown dtype or algorithm code */
    W4A8_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned */
    W4A8_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than required */
    W4A8_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed */
    W4A8_ERR_DEVICE = 7      /* the current device is not a gfx950 (MI355X-class) GPU */
} w4a8_status;

/* Element types of floating-point inputs and outputs. */
typedef enum { W4A8_F32 = 0, W4A8_BF16 = 1 } w4a8_dtype;

/* Kernel choice for w4a8_linear_algo. */
typedef enum {
    W4A8_ALGO_AUTO = 0,       /* pick by M, N, K (what w4a8_linear does): GEMV within its
                                 range for M <= 3, SKINNY for M <= 64, else MFMA_F16 */
    W4A8_ALGO_GEMV = 1,       /* streaming GEMV (decode); M <= 4 and M*K <= 40960.  The
                                 codebook is read as fp16 pairs (two levels per packed byte),
                                 each level scaled by the power of two that brings the largest
                                 into [0.5, 1) and rounded to fp16: a relative error of at most
                                 2^-11 per level (levels under 2^-14 of the largest: an absolute
                                 error of at most 2^-25 of that power of two), fp32 sums */
    W4A8_ALGO_MFMA_I8 = 2,    /* the int8 form of the codebook, cb_i8 = rint(codebook / s_cb),
                                 s_cb = max|codebook| / 127.  Each weight cb_i8[idx] * dec(s_rel)
                                 is exact in fp16 (at most 11 significant bits, 2^-9 to 56896)
                                 and each product with x_q exact in fp32, so a group's products
                                 sum to its exact int8 partial times its group scale; f16 MFMA,
                                 fp32 accumulation, y = acc * s_cb * s_channel * s_x (the same
                                 tiles as MFMA_F16).  Each level moves by up to s_cb / 2: on top
                                 of the fp32 accumulation the output carries up to
                                 s_x * s_channel * sum_g |dec(s_rel)| *
                                 (s_cb / 2) * sum_{k in g} |x_q|.  That term is not inside the
                                 4e-3 bound of w4a8_linear for every input (activations that
                                 fall on small levels only can exceed it); dense activations
                                 meet the bound with a wide margin.  An explicit choice, never
                                 the automatic one */
    W4A8_ALGO_MFMA_F16 = 3,   /* f16 MFMA on decoded weights: fp16(codebook level x 2^-ex) times
                                 fp16(dec(s_rel) x 2^7) rounded to fp16 (at most 2^-10 relative
                                 per weight), fp32 accumulation; one workgroup per tile of
                                 256 tokens x 192 rows (64 x 64 up to 64 tokens, 32 x 64 up to
                                 32) */
    W4A8_ALGO_MFMA_SKINNY = 4, /* the same numerics as MFMA_F16 for M <= 64 (batched decode):
                                 16-row weight tiles streamed once, M*K < 2^31 */
    W4A8_ALGO_MFMA_RQ = 5,    /* full-rate int8 MFMA on requantised weights (prefill):
                                 q = rint(dec(s_rel) * codebook[idx] / s_cb), s_cb = max|codebook|
                                 / 127, clamped to +-127, one int32 sum per output,
                                 y = ((float)sum * (s_channel * s_cb)) * s_x; K <= 131072.
                                 Weight rounding to the step s_cb is the only approximation
                                 (card A "Why this exists": int8 GEMM + dequantisation step);
                                 like MFMA_I8 an explicit choice whose error is not inside the
                                 4e-3 bound for every input */
    W4A8_ALGO_MFMA_I8_FOLD = 6 /* the int8-codebook product computed step by step as the int8
                                 path is described: v_mfma_i32_32x32x16_i8 (K = 16, one group)
                                 gives the exact int32 partial P = sum x_q * cb_i8[idx] of each
                                 group, and the vector ALU folds it, acc = fma(dec(s_rel),
                                 (float)P, acc), group by group; y = acc * s_cb * s_channel *
                                 s_x.  The same numerics as MFMA_I8 up to the order of the fp32
                                 additions (identical bits on most outputs, a few ulps apart on
                                 the rest), at roughly 0.6x its rate: the fold's conversion and
                                 fma per partial run on the vector ALU.  256 x 192 tiles.  An
                                 explicit choice */
} w4a8_algo;

/* Library version: major * 10000 + minor * 100 + patch. */
W4A8_API int w4a8_version(void);

/* Human-readable text of a status code (static storage; never NULL). */
W4A8_API const char *w4a8_status_string(int status);

/*
 * Bytes of device workspace w4a8_quantize_weight needs for an N x K weight (0 if the shape
 * is invalid): the fit sample's keys and prefix sums, at most 12,583,168 bytes whatever the
 * shape.
 */
W4A8_API size_t w4a8_quantize_weight_workspace(int64_t N, int64_t K);

/*
 * Offline quantisation of one weight matrix into the four-tensor layer format
 * [card "...w4a8-convrot-ComfyUI", sections "Format" and "Reproducing"; card
 * "Qwen3.8-27B-W4A8", section "Model Overview": Hadamard rotation in 256-blocks, then
 * group quantisation with a 16-level Lloyd-Max codebook, fp8 group scales and fp32
 * channel scales; the seed pins the codebook fit, which samples].
 *
 *  w          [N][K] weights, element type w_dtype (W4A8_F32 or W4A8_BF16)
 *  N, K       N >= 1; K >= 256 and K % 256 == 0 (the rotation block must divide K)
 *  seed       seeds the SplitMix64 draw of the 2^20-value fit sample (used when N*K > 2^20)
 *  packed, s_rel, s_channel, codebook   outputs, layouts as above; codebook ascending
 *  workspace  device scratch of at least w4a8_quantize_weight_workspace(N, K) bytes
 *
 * Steps (all on the device, in stream order): rotate each row by 256-blocks;
 * s_channel = row max |w_rot|; s_rel = E4M3FN(group max |w_rot| / s_channel), round to
 * nearest even; v = w_rot / (s_channel * dec(s_rel)); fit 16 levels to v by Lloyd's
 * iteration in fp64 (mid-quantile start, at most 100 updates); each element takes its
 * nearest level (ties to the lower index); pack.  Deterministic in (w, N, K, seed).
 */
W4A8_API int w4a8_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, uint64_t seed,
                         int8_t *packed, uint8_t *s_rel, float *s_channel, float *codebook,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a8_quantize_weight for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): the same kernels and the same
 * results, bit for bit, with the workspace in a static device array of the library, so the
 * caller passes no workspace and the call allocates nothing.
 *
 *  Arguments as for w4a8_quantize_weight, without workspace / workspace_bytes.
 *  Scratch: 12,583,168 bytes per device (the workspace of a full 2^20-value fit sample, the
 *  most any N x K needs), held by each device the library runs on until the process ends.
 *  A shape whose workspace would exceed it returns W4A8_ERR_WORKSPACE (none does today).
 *  Every call on one device shares that device's array and leaves its contents behind (the
 *  kernels overwrite all of it that they read), so calls that overlap on one device -- on
 *  different streams or from different threads -- race and must be serialised by the caller.
 */
W4A8_API int w4a8_quantize_weight_noalloc(const void *w, int w_dtype, int64_t N, int64_t K, uint64_t seed,
                                          int8_t *packed, uint8_t *s_rel, float *s_channel, float *codebook,
                                          void *stream);

/*
 * Per-call activation preparation [card "Qwen3.8-27B-W4A8", section "Model Overview":
 * 4-bit weights with int8 activations; card "...w4a8-convrot-ComfyUI", section "Format":
 * the layer executes on int8 GEMM in the rotated basis].
 *
 *  x      [M][K] activations, element type x_dtype (W4A8_F32 or W4A8_BF16)
 *  M, K   M >= 1; K >= 256 and K % 256 == 0
 *  x_q    [M][K] int8 output;  s_x  [M] fp32 output
 *
 * Each 256-block of each row is rotated (fp32 fast Hadamard transform, stages of span
 * 1, 2, ..., 128 in that order, then x 1/16); then per row amax = max |x_rot|,
 * s_x = amax / 127 and x_q = clamp(rint(x_rot / s_x), -127, 127) with IEEE division and
 * ties to even; an all-zero row gives s_x = 0 and x_q = 0.  Results are bit-exact and
 * deterministic.
 */
W4A8_API int w4a8_prepare_activation(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *x_q,
                            float *s_x, void *stream);

/*
 * The quantised product [card "...w4a8-convrot-ComfyUI", sections "Why this exists"
 * and "Format": the layer runs on the int8 GEMM path with a codebook dequantisation step
 * on top; a weight is its codebook level times its group's scale times its row's scale].
 *
 *  x_q, s_x   prepared activations [M][K], [M] (from w4a8_prepare_activation)
 *  packed, s_rel, s_channel, codebook   one layer, layouts as above, N rows
 *  y          [M][N] output, element type y_dtype (W4A8_F32 or W4A8_BF16)
 *  M >= 1, N >= 1, K >= 256, K % 256 == 0
 *
 * Each output satisfies |y - y_exact| <= 4e-3 * sum_k |s_x x_q[k] w_hat[k]| where y_exact
 * is the fp64 value of the formula above (bf16 output adds its own rounding), for any group
 * scale byte except the two NaN codes (0x7F, 0xFF), and for codebook levels no smaller in
 * magnitude than 2^-12 of the largest (the fp16 forms of smaller levels carry an absolute
 * rather than a relative error; such levels contribute correspondingly little).  Output
 * is deterministic: no atomics, fixed reduction order for a given (M, N, K, algorithm).
 */
W4A8_API int w4a8_linear(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *packed,
                const uint8_t *s_rel, const float *s_channel, const float *codebook, int64_t N,
                void *y, int y_dtype, void *stream);

/* As w4a8_linear with an explicit kernel choice (w4a8_algo).  W4A8_ALGO_GEMV returns
 * W4A8_ERR_SHAPE outside its range (M <= 4 and M*K <= 40960), W4A8_ALGO_MFMA_SKINNY outside
 * its range (M <= 64, M*K < 2^31, 40*K < 2^31), W4A8_ALGO_MFMA_RQ for K > 131072 (the
 * int32 sum must stay exact), and the four prefill GEMMs (MFMA_I8, MFMA_F16, MFMA_RQ,
 * MFMA_I8_FOLD) for more than 2^31 - 1 workgroup tiles (see the algorithm list for the tile
 * shapes).  An unknown algorithm code returns W4A8_ERR_DTYPE. */
W4A8_API int w4a8_linear_algo(const int8_t *x_q, const float *s_x, int64_t M, int64_t K,
                     const int8_t *packed, const uint8_t *s_rel, const float *s_channel,
                     const float *codebook, int64_t N, void *y, int y_dtype, int algo,
                     void *stream);

/*
 * Activation preparation and product in one call: the same results as
 * w4a8_prepare_activation(x -> x_q, s_x) followed by w4a8_linear(x_q, s_x -> y), bit for
 * bit in x_q and s_x and within the same bound in y.  For decode sizes (M = 1 with
 * K <= 32768, or M = 2 with K <= 20480) both run in ONE kernel launch: the GEMV's
 * workgroups rotate and quantise
 * the activations in their prologue [card "...w4a8-convrot-ComfyUI", section "Why this
 * exists": every generated token re-reads all weights, so per-token fixed costs matter];
 * otherwise the two steps run as separate launches.  x_q [M][K] and s_x [M] are
 * caller-provided outputs in both cases.  Argument rules as for the two calls.
 */
W4A8_API int w4a8_forward(const void *x, int x_dtype, int64_t M, int64_t K, const int8_t *packed,
                          const uint8_t *s_rel, const float *s_channel, const float *codebook,
                          int64_t N, void *y, int y_dtype, int8_t *x_q, float *s_x, void *stream);

/*
 * Workspace bytes w4a8_linear_ws can use for (M, N, K) on the current device, or 0 when the
 * algorithm w4a8_linear picks needs none (a negative status for an invalid shape).  Only
 * the batched-decode kernel uses one, from 17 to 64 tokens: where a workgroup would own few
 * rows (under 80 per compute unit, as for the MLP down projection) and K is long (a multiple
 * of 1024, at least 8192), it splits K into 4 parts, each workgroup taking full row tiles
 * over one part, so that every compute unit reads a quarter of the activations.  Launches
 * nothing.
 */
W4A8_API int64_t w4a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * w4a8_linear with a workspace [the same product and card sections as w4a8_linear].
 *
 *  workspace        device memory, 16-byte aligned, of workspace_bytes bytes: 4 KiB of
 *                   arrival counters, then the parts' sums.  It must be zero-filled before
 *                   its first use; every call that completes leaves the counters at zero, so
 *                   one workspace serves any later shape it is large enough for.  Calls that
 *                   overlap in time (other streams, other threads) need workspaces of their
 *                   own.
 *  workspace_bytes  at least w4a8_linear_workspace_bytes(M, N, K) to split K; with less (or
 *                   a NULL workspace) the call runs exactly as w4a8_linear.
 *
 * With the split, each part's workgroup stores its partial sums (fp32, before the row and
 * token scales) in the workspace and counts its arrival on an atomic counter of its row
 * block; the last part to arrive adds the parts' sums in part order, scales them and
 * writes y.  The result depends on the part order only, not on the order of arrival, so it
 * is deterministic; it differs from w4a8_linear's only by the order of fp32 additions and
 * meets the same bound.
 */
W4A8_API int w4a8_linear_ws(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *packed,
                            const uint8_t *s_rel, const float *s_channel, const float *codebook, int64_t N,
                            void *y, int y_dtype, void *workspace, int64_t workspace_bytes, void *stream);

/* The algorithm w4a8_linear picks for (M, N, K) on the current device, or a negative
 * status if the shape is invalid.  Launches nothing. */
W4A8_API int w4a8_linear_pick(int64_t M, int64_t N, int64_t K);

/*
 * One quantised layer for the multi-layer calls below: its four tensors, its row count and
 * its output [M][N].  Device pointers, as everywhere.
 */
typedef struct {
    const int8_t *packed;       /* [N][K/2] */
    const uint8_t *s_rel;       /* [N][K/16] */
    const float *s_channel;     /* [N] */
    const float *codebook;      /* [16] */
    int64_t N;                  /* rows, >= 1 */
    void *y;                    /* [M][N] output, element type y_dtype */
} w4a8_layer;

/*
 * Several layers that read the same activations (the query/key/value projections of one
 * input, or gate and up) in one call [card "...w4a8-convrot-ComfyUI", section "Why this
 * exists": decode re-reads every weight for every token, so each launch's fixed cost is paid
 * once per layer per token].  Where w4a8_linear takes the GEMV (M <= 3 and M*K <= 40960)
 * all layers run in ONE launch, its workgroups split between the layers in proportion to their rows.
 * Where it takes the batched-decode kernel and all layers have the same N, they also run in
 * one launch, each workgroup doing what the single-layer launch does for its rows.
 * Otherwise each layer runs as w4a8_linear would.  Every y is bit-identical to what
 * w4a8_linear gives for that layer alone.
 *
 *  layers   HOST array of G descriptors, 1 <= G <= 8; read during the call only
 *  others   as for w4a8_linear; each layer is validated like a w4a8_linear call
 */
W4A8_API int w4a8_linear_multi(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, int G,
                               const w4a8_layer *layers, int y_dtype, void *stream);

/*
 * Activation preparation and several layers in one call: the results of
 * w4a8_prepare_activation followed by w4a8_linear_multi, bit for bit.  For the fused decode
 * sizes of w4a8_forward everything runs in ONE launch.  x_q [M][K] and s_x [M] are outputs.
 */
W4A8_API int w4a8_forward_multi(const void *x, int x_dtype, int64_t M, int64_t K, int G,
                                const w4a8_layer *layers, int y_dtype, int8_t *x_q, float *s_x,
                                void *stream);

/*
 * W8A8 comparator: the "INT8 ConvRot" build the W4A8 format is weighed against [card
 * "...w4a8-convrot-ComfyUI", section "Why this exists": an INT8 ConvRot build of the model
 * takes about twice the weight bytes, and W4A8 runs on the same int8 GEMM path plus a
 * codebook dequantisation step].  Same rotation and int8 activations as above; the weights
 * are int8 with one fp32 scale per row and no codebook or group scales.  The pages fix no
 * more than that; the per-row scale is the plainest reading beside the per-token one.
 *
 * Weight quantisation: each row of w [N][K] (element type w_dtype) is rotated and quantised
 * exactly as w4a8_prepare_activation treats a token: s_w[r] = max |w_rot[r]| / 127 and
 * w_q[r][k] = clamp(rint(w_rot[r][k] / s_w[r]), -127, 127); a zero row gives 0.
 *  w_q [N][K] int8, s_w [N] fp32: outputs.   N >= 1; 256 <= K <= 131072, K % 256 == 0.
 */
W4A8_API int w4a8_w8a8_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, int8_t *w_q,
                                       float *s_w, void *stream);

/*
 * W8A8 product: y[m][r] = (fp32(sum_k x_q[m][k] * w_q[r][k]) * s_w[r]) * s_x[m], the integer
 * sum exact in int32 and each product one fp32 rounding, so |y - y_exact| <= 4 * 2^-24 *
 * |y_exact| (bf16 output adds its own rounding).  Deterministic.
 *
 *  x_q, s_x   prepared activations [M][K], [M];  w_q, s_w  [N][K], [N] (as quantised above)
 *  y          [M][N], element type y_dtype;  M, N >= 1; 256 <= K <= 131072, K % 256 == 0
 *  algo       W4A8_ALGO_AUTO (GEMV when M <= 4 and M*K <= 65536, else MFMA_I8),
 *             W4A8_ALGO_GEMV (W4A8_ERR_SHAPE outside that range) or W4A8_ALGO_MFMA_I8 (int8
 *             MFMA GEMM, any M); any other code is W4A8_ERR_DTYPE.
 */
W4A8_API int w4a8_w8a8_linear(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *w_q,
                              const float *s_w, int64_t N, void *y, int y_dtype, int algo, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
