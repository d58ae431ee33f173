// C ABI of libw4a8.so: argument validation, device check and kernel dispatch.
// The public contract (layouts, semantics, error behaviour) is stated in include/w4a8.h.
#include <string.h>

#include <atomic>

#include "../../include/w4a8.h"
#include "w4a8_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// per device: 0 = unknown, 1 = gfx950, 2 = other; CU count cached beside it
std::atomic<int> g_dev_kind[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

// Resolve the current device once: it must be a gfx950.  Returns a w4a8_status.
int current_device(int *num_cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return W4A8_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return W4A8_ERR_DEVICE;
    int kind = g_dev_kind[dev].load(std::memory_order_acquire);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return W4A8_ERR_HIP;
        kind = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_dev_kind[dev].store(kind, std::memory_order_release);
    }
    if (kind != 1) return W4A8_ERR_DEVICE;
    if (num_cu) *num_cu = g_dev_cus[dev].load(std::memory_order_relaxed);
    return W4A8_OK;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_k(int64_t K) { return K >= 256 && K % 256 == 0 && K <= (int64_t(1) << 30); }
inline bool valid_dtype(int d) { return d == W4A8_F32 || d == W4A8_BF16; }

int check_linear(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *packed,
                 const uint8_t *s_rel, const float *s_channel, const float *codebook, int64_t N,
                 void *y, int y_dtype) {
    if (!x_q || !s_x || !packed || !s_rel || !s_channel || !codebook || !y) return W4A8_ERR_NULL;
    if (M < 1 || N < 1 || !valid_k(K) || M > (int64_t(1) << 31) - 1 || N > (int64_t(1) << 31) - 1)
        return W4A8_ERR_SHAPE;
    if (!valid_dtype(y_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(x_q) || !aligned16(s_x) || !aligned16(packed) || !aligned16(s_rel) ||
        !aligned16(s_channel) || !aligned16(codebook) || !aligned16(y))
        return W4A8_ERR_ALIGN;
    return W4A8_OK;
}

// Where w4a8_linear takes the GEMV: within its range up to M = 3; from M = 4 the skinny
// kernel is faster (measured crossover).  The multi-layer call follows the same rule so that
// its outputs stay bit-identical to single-layer calls.
inline bool gemv_auto(int64_t M, int64_t K) { return w4a8::gemv_supported(M, K) && M <= 3; }

int pick(int64_t M, int64_t N, int64_t K) {
    if (gemv_auto(M, K)) return W4A8_ALGO_GEMV;
    if (w4a8::skinny_supported(M, N, K)) return W4A8_ALGO_MFMA_SKINNY;
    return W4A8_ALGO_MFMA_F16;
}

}  // namespace

extern "C" {

int w4a8_version(void) { return 100; }

const char *w4a8_status_string(int status) {
    switch (status) {
        case W4A8_OK: return "ok";
        case W4A8_ERR_NULL: return "a required pointer is NULL";
        case W4A8_ERR_SHAPE: return "invalid shape (M, N >= 1; K >= 256 and a multiple of 256)";
        case W4A8_ERR_DTYPE: return "unknown dtype or algorithm code";
        case W4A8_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case W4A8_ERR_WORKSPACE: return "workspace missing or too small";
        case W4A8_ERR_HIP: return "HIP runtime call or kernel launch failed";
        case W4A8_ERR_DEVICE: return "current device is not a gfx950 GPU";
        default: return "unknown status";
    }
}

size_t w4a8_quantize_weight_workspace(int64_t N, int64_t K) {
    if (N < 1 || !valid_k(K) || N > (int64_t(1) << 31) - 1) return 0;
    return w4a8::quantize_workspace_bytes(N, K);
}

int w4a8_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, uint64_t seed,
                         int8_t *packed, uint8_t *s_rel, float *s_channel, float *codebook,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (!w || !packed || !s_rel || !s_channel || !codebook) return W4A8_ERR_NULL;
    if (N < 1 || !valid_k(K) || N > (int64_t(1) << 31) - 1) return W4A8_ERR_SHAPE;
    if (!valid_dtype(w_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(s_rel) || !aligned16(s_channel) ||
        !aligned16(codebook))
        return W4A8_ERR_ALIGN;
    if (!workspace || workspace_bytes < w4a8::quantize_workspace_bytes(N, K)) return W4A8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return W4A8_ERR_ALIGN;
    int st = current_device(nullptr);
    if (st != W4A8_OK) return st;
    hipError_t e = w4a8::launch_quantize(w, w_dtype == W4A8_BF16, N, K, seed, packed, s_rel, s_channel,
                                         codebook, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_quantize_weight_noalloc(const void *w, int w_dtype, int64_t N, int64_t K, uint64_t seed,
                                 int8_t *packed, uint8_t *s_rel, float *s_channel, float *codebook,
                                 void *stream) {
    if (!w || !packed || !s_rel || !s_channel || !codebook) return W4A8_ERR_NULL;
    if (N < 1 || !valid_k(K) || N > (int64_t(1) << 31) - 1) return W4A8_ERR_SHAPE;
    if (!valid_dtype(w_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(s_rel) || !aligned16(s_channel) ||
        !aligned16(codebook))
        return W4A8_ERR_ALIGN;
    int st = current_device(nullptr);
    if (st != W4A8_OK) return st;
    void *ws = nullptr;
    size_t cap = 0;
    if (w4a8::quantize_scratch(&ws, &cap) != hipSuccess) return W4A8_ERR_HIP;
    if (w4a8::quantize_workspace_bytes(N, K) > cap) return W4A8_ERR_WORKSPACE;
    hipError_t e = w4a8::launch_quantize(w, w_dtype == W4A8_BF16, N, K, seed, packed, s_rel, s_channel,
                                         codebook, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_prepare_activation(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *x_q,
                            float *s_x, void *stream) {
    if (!x || !x_q || !s_x) return W4A8_ERR_NULL;
    if (M < 1 || !valid_k(K) || M > (int64_t(1) << 31) - 1) return W4A8_ERR_SHAPE;
    if (!valid_dtype(x_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(x_q) || !aligned16(s_x)) return W4A8_ERR_ALIGN;
    int num_cu = 0;
    int st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    hipError_t e = w4a8::launch_prepare(x, x_dtype == W4A8_BF16, M, K, x_q, s_x, num_cu,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_linear_pick(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || !valid_k(K)) return -W4A8_ERR_SHAPE;
    return pick(M, N, K);
}

int w4a8_linear_algo(const int8_t *x_q, const float *s_x, int64_t M, int64_t K,
                     const int8_t *packed, const uint8_t *s_rel, const float *s_channel,
                     const float *codebook, int64_t N, void *y, int y_dtype, int algo,
                     void *stream) {
    int st = check_linear(x_q, s_x, M, K, packed, s_rel, s_channel, codebook, N, y, y_dtype);
    if (st != W4A8_OK) return st;
    if (algo == W4A8_ALGO_AUTO) algo = pick(M, N, K);
    if (algo != W4A8_ALGO_GEMV && algo != W4A8_ALGO_MFMA_I8 && algo != W4A8_ALGO_MFMA_F16 &&
        algo != W4A8_ALGO_MFMA_SKINNY && algo != W4A8_ALGO_MFMA_RQ && algo != W4A8_ALGO_MFMA_I8_FOLD)
        return W4A8_ERR_DTYPE;
    if (algo == W4A8_ALGO_GEMV && !w4a8::gemv_supported(M, K)) return W4A8_ERR_SHAPE;
    if (algo == W4A8_ALGO_MFMA_SKINNY && !w4a8::skinny_supported(M, N, K)) return W4A8_ERR_SHAPE;
    if (algo == W4A8_ALGO_MFMA_RQ && !w4a8::gemm_rq_supported(M, N, K)) return W4A8_ERR_SHAPE;
    // the decoded-weight GEMMs launch one workgroup per tile (256 x 192, or smaller tiles for
    // few tokens)
    if ((algo == W4A8_ALGO_MFMA_I8 || algo == W4A8_ALGO_MFMA_F16) && !w4a8::gemm_dec_tiles_fit(M, N))
        return W4A8_ERR_SHAPE;
    if (algo == W4A8_ALGO_MFMA_I8_FOLD && ((M + 255) / 256) * ((N + 191) / 192) > (int64_t(1) << 31) - 1)
        return W4A8_ERR_SHAPE;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    w4a8::LinearArgs a{x_q, s_x, M, K, N, packed, s_rel, s_channel, codebook, y, y_dtype == W4A8_BF16,
                       nullptr, 0, nullptr, nullptr};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (algo) {
        case W4A8_ALGO_GEMV: e = w4a8::launch_gemv(a, num_cu, s); break;
        case W4A8_ALGO_MFMA_I8: e = w4a8::launch_gemm_i8(a, s); break;
        case W4A8_ALGO_MFMA_SKINNY: e = w4a8::launch_gemm_skinny(a, num_cu, s); break;
        case W4A8_ALGO_MFMA_RQ: e = w4a8::launch_gemm_rq(a, s); break;
        case W4A8_ALGO_MFMA_I8_FOLD: e = w4a8::launch_gemm_i8_fold(a, s); break;
        default: e = w4a8::launch_gemm_f16(a, s); break;
    }
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_forward(const void *x, int x_dtype, int64_t M, int64_t K, const int8_t *packed,
                 const uint8_t *s_rel, const float *s_channel, const float *codebook, int64_t N,
                 void *y, int y_dtype, int8_t *x_q, float *s_x, void *stream) {
    if (!x) return W4A8_ERR_NULL;
    int st = check_linear(x_q, s_x, M, K, packed, s_rel, s_channel, codebook, N, y, y_dtype);
    if (st != W4A8_OK) return st;
    if (!valid_dtype(x_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(x)) return W4A8_ERR_ALIGN;
    if (!(w4a8::gemv_fused_supported(M, K) && pick(M, N, K) == W4A8_ALGO_GEMV)) {
        st = w4a8_prepare_activation(x, x_dtype, M, K, x_q, s_x, stream);
        if (st != W4A8_OK) return st;
        return w4a8_linear(x_q, s_x, M, K, packed, s_rel, s_channel, codebook, N, y, y_dtype, stream);
    }
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    w4a8::LinearArgs a{x_q, s_x, M, K, N, packed, s_rel, s_channel, codebook, y, y_dtype == W4A8_BF16,
                       x, x_dtype == W4A8_BF16, x_q, s_x};
    hipError_t e = w4a8::launch_gemv_fused(a, num_cu, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

// Validates G and every layer; fills the internal descriptors.
static int check_multi(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, int G,
                       const w4a8_layer *layers, int y_dtype, w4a8::LayerDesc *out) {
    if (!layers) return W4A8_ERR_NULL;
    if (G < 1 || G > w4a8::kMaxGroup) return W4A8_ERR_SHAPE;
    for (int g = 0; g < G; g++) {
        const w4a8_layer &l = layers[g];
        int st = check_linear(x_q, s_x, M, K, l.packed, l.s_rel, l.s_channel, l.codebook, l.N, l.y, y_dtype);
        if (st != W4A8_OK) return st;
        out[g] = w4a8::LayerDesc{l.packed, l.s_rel, l.s_channel, l.codebook, l.N, l.y};
    }
    return W4A8_OK;
}

int w4a8_linear_multi(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, int G,
                      const w4a8_layer *layers, int y_dtype, void *stream) {
    w4a8::LayerDesc d[w4a8::kMaxGroup];
    int st = check_multi(x_q, s_x, M, K, G, layers, y_dtype, d);
    if (st != W4A8_OK) return st;
    if (!gemv_auto(M, K)) {
        // layers of one row count on the batched-decode kernel: one launch, each workgroup
        // running what the single-layer launch runs for its rows
        bool same_n = G > 1;
        for (int g = 1; g < G; g++) same_n = same_n && d[g].N == d[0].N;
        if (same_n && pick(M, d[0].N, K) == W4A8_ALGO_MFMA_SKINNY) {
            int num_cu = 0;
            st = current_device(&num_cu);
            if (st != W4A8_OK) return st;
            w4a8::LinearArgs a{x_q, s_x, M, K, d[0].N, d[0].packed, d[0].s_rel, d[0].s_ch, d[0].cb, d[0].y,
                               y_dtype == W4A8_BF16, nullptr, 0, nullptr, nullptr};
            hipError_t e = w4a8::launch_gemm_skinny_multi(a, d, G, num_cu, static_cast<hipStream_t>(stream));
            return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
        }
        for (int g = 0; g < G; g++) {
            st = w4a8_linear(x_q, s_x, M, K, d[g].packed, d[g].s_rel, d[g].s_ch, d[g].cb, d[g].N, d[g].y,
                             y_dtype, stream);
            if (st != W4A8_OK) return st;
        }
        return W4A8_OK;
    }
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    w4a8::LinearArgs a{x_q, s_x, M, K, 0, nullptr, nullptr, nullptr, nullptr, nullptr, y_dtype == W4A8_BF16,
                       nullptr, 0, nullptr, nullptr};
    hipError_t e = w4a8::launch_gemv_multi(a, d, G, num_cu, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_forward_multi(const void *x, int x_dtype, int64_t M, int64_t K, int G, const w4a8_layer *layers,
                       int y_dtype, int8_t *x_q, float *s_x, void *stream) {
    if (!x) return W4A8_ERR_NULL;
    w4a8::LayerDesc d[w4a8::kMaxGroup];
    int st = check_multi(x_q, s_x, M, K, G, layers, y_dtype, d);
    if (st != W4A8_OK) return st;
    if (!valid_dtype(x_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(x)) return W4A8_ERR_ALIGN;
    if (!w4a8::gemv_fused_supported(M, K)) {
        st = w4a8_prepare_activation(x, x_dtype, M, K, x_q, s_x, stream);
        if (st != W4A8_OK) return st;
        return w4a8_linear_multi(x_q, s_x, M, K, G, layers, y_dtype, stream);
    }
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    w4a8::LinearArgs a{x_q, s_x, M, K, 0, nullptr, nullptr, nullptr, nullptr, nullptr, y_dtype == W4A8_BF16,
                       x, x_dtype == W4A8_BF16, x_q, s_x};
    hipError_t e = w4a8::launch_gemv_fused_multi(a, d, G, num_cu, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_w8a8_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, int8_t *w_q,
                              float *s_w, void *stream) {
    if (!w || !w_q || !s_w) return W4A8_ERR_NULL;
    if (N < 1 || !valid_k(K) || K > w4a8::kW8MaxK || N > (int64_t(1) << 31) - 1) return W4A8_ERR_SHAPE;
    if (!valid_dtype(w_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(w) || !aligned16(w_q) || !aligned16(s_w)) return W4A8_ERR_ALIGN;
    int num_cu = 0;
    int st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    // a weight row is quantised exactly as a token is: rotate, per-row max / 127, round
    hipError_t e = w4a8::launch_prepare(w, w_dtype == W4A8_BF16, N, K, w_q, s_w, num_cu,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_w8a8_linear(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *w_q,
                     const float *s_w, int64_t N, void *y, int y_dtype, int algo, void *stream) {
    if (!x_q || !s_x || !w_q || !s_w || !y) return W4A8_ERR_NULL;
    if (M < 1 || N < 1 || !valid_k(K) || K > w4a8::kW8MaxK || M > (int64_t(1) << 31) - 1 ||
        N > (int64_t(1) << 31) - 1)
        return W4A8_ERR_SHAPE;
    if (!valid_dtype(y_dtype)) return W4A8_ERR_DTYPE;
    if (!aligned16(x_q) || !aligned16(s_x) || !aligned16(w_q) || !aligned16(s_w) || !aligned16(y))
        return W4A8_ERR_ALIGN;
    if (algo == W4A8_ALGO_AUTO) algo = w4a8::w8_gemv_supported(M, K) ? W4A8_ALGO_GEMV : W4A8_ALGO_MFMA_I8;
    if (algo != W4A8_ALGO_GEMV && algo != W4A8_ALGO_MFMA_I8) return W4A8_ERR_DTYPE;
    if (algo == W4A8_ALGO_GEMV && !w4a8::w8_gemv_supported(M, K)) return W4A8_ERR_SHAPE;
    // the tile count must fit the grid
    if (algo == W4A8_ALGO_MFMA_I8 && ((M + 255) / 256) * ((N + 191) / 192) > (int64_t(1) << 31) - 1)
        return W4A8_ERR_SHAPE;
    int num_cu = 0;
    int st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    w4a8::W8Args a{x_q, s_x, M, K, N, w_q, s_w, y, y_dtype == W4A8_BF16};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = algo == W4A8_ALGO_GEMV ? w4a8::launch_w8_gemv(a, num_cu, s) : w4a8::launch_w8_gemm(a, s);
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int64_t w4a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || !valid_k(K)) return -W4A8_ERR_SHAPE;
    if (pick(M, N, K) != W4A8_ALGO_MFMA_SKINNY) return 0;
    int num_cu = 0;
    int st = current_device(&num_cu);
    if (st != W4A8_OK) return -st;
    return w4a8::skinny_workspace_bytes(M, N, K, num_cu);
}

int w4a8_linear_ws(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *packed,
                   const uint8_t *s_rel, const float *s_channel, const float *codebook, int64_t N,
                   void *y, int y_dtype, void *workspace, int64_t workspace_bytes, void *stream) {
    int st = check_linear(x_q, s_x, M, K, packed, s_rel, s_channel, codebook, N, y, y_dtype);
    if (st != W4A8_OK) return st;
    if (workspace && !aligned16(workspace)) return W4A8_ERR_ALIGN;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A8_OK) return st;
    const int64_t need = pick(M, N, K) == W4A8_ALGO_MFMA_SKINNY ? w4a8::skinny_workspace_bytes(M, N, K, num_cu) : 0;
    if (need == 0 || !workspace || workspace_bytes < need)
        return w4a8_linear_algo(x_q, s_x, M, K, packed, s_rel, s_channel, codebook, N, y, y_dtype,
                                W4A8_ALGO_AUTO, stream);
    const int q = w4a8::skinny_split(M, N, K, num_cu);
    w4a8::LinearArgs a{x_q, s_x, M, K, N, packed, s_rel, s_channel, codebook, y, y_dtype == W4A8_BF16,
                       nullptr, 0, nullptr, nullptr};
    a.ksplit = q;
    a.ws_cnt = static_cast<uint32_t *>(workspace);
    a.ws_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + w4a8::kSkinnyCounterBytes);
    hipError_t e = w4a8::launch_gemm_skinny(a, num_cu, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A8_OK : W4A8_ERR_HIP;
}

int w4a8_linear(const int8_t *x_q, const float *s_x, int64_t M, int64_t K, const int8_t *packed,
                const uint8_t *s_rel, const float *s_channel, const float *codebook, int64_t N,
                void *y, int y_dtype, void *stream) {
    return w4a8_linear_algo(x_q, s_x, M, K, packed, s_rel, s_channel, codebook, N, y, y_dtype,
                            W4A8_ALGO_AUTO, stream);
}

}  // extern "C"
