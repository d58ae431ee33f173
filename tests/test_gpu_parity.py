"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Integers -- packed indices, e4m3 group-scale bytes, row scales, codebook bits, int8
activations and their scales -- must match bit for bit.  Products must satisfy
|y - y_ref| <= 4e-3 * A with y_ref and A = sum_k |s_x x_q w_hat| from the oracle's fp64
definition; the int8-codebook route must also match the oracle's int8-codebook value y8
within (G + 4) * 2^-24 * A8 for G = K/16 groups (the fp32 rounding of one addition per group
of 16 exact products, plus the epilogue's).  Full-size
shapes are checked on sampled rows and tokens; small shapes span several tiles and ragged
tails in full.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_codebook_gemm_amd as mod
    mod.lib()
    return mod


DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@functools.lru_cache(maxsize=None)
def oracle_layer(N, K, seed=0):
    W = S.weights(N, K, seed=seed)
    return W, O.quantize_weight(W, seed=seed)


@functools.lru_cache(maxsize=None)
def oracle_acts(M, K, seed=0, n_out=None):
    x = S.activations(M, K, seed=seed, n_outliers=n_out)
    xq, sx = O.prepare(x)
    return x, xq, sx


def gpu_layer(w, q):
    return w.QuantizedLinear(gpu(q["packed"]), gpu(q["s_rel"]), gpu(q["s_ch"]), gpu(q["cb"]))


def sample(n, count, seed):
    if n <= count:
        return np.arange(n)
    r = S.u64(seed, 77, count) % np.uint64(n)
    return np.unique(np.concatenate([[0, n - 1], r.astype(np.int64)]))


# ----------------------------------------------------------------------------- prepare

# K from one block (one 64-thread workgroup) through two register rounds (K <= 32768) to the
# two-pass path for longer rows; the two fp32 prefill launches the benchmark times (2048 tokens
# of the MLP input and of the hidden activation) are included as they are timed
PREP_CASES = [(4, 512, "f32"), (4, 512, "bf16"), (1, 256, "f32"), (3, 5120, "f32"),
              (2, 17408, "bf16"), (37, 768, "f32"), (5, 20736, "f32"), (2048, 5120, "bf16"),
              (2048, 5120, "f32"), (2048, 17408, "f32"),
              (3, 32768, "f32"), (3, 33024, "bf16"), (2, 65536, "f32")]


@pytest.mark.parametrize("M,K,dt", PREP_CASES)
def test_prepare_bit_exact(w, M, K, dt):
    say(f"prepare M={M} K={K} {dt}")
    x = S.activations(M, K, seed=M + K, n_outliers=2)
    if M > 2:
        x[1] = 0.0                      # all-zero token
        x[2] = 0.0
        x[2, K // 3] = -3.0             # a single spike
    if dt == "bf16":
        bits = S.to_bf16_bits(x)
        xin = gpu(bits.view(np.int16)).view(torch.bfloat16)
        x = S.bf16_bits_to_f32(bits)
    else:
        xin = gpu(x)
    xq_ref, sx_ref = O.prepare(x)
    xq, sx = w.prepare_activation(xin)
    torch.cuda.synchronize()
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("fused", [False, True])
def test_prepare_tiny_scales(w, fused):
    """Both quantisation routes: ordinary scales (reciprocal with exact correction) and
    s_x below 2^-100 (IEEE division), including a token of subnormal values."""
    say(f"prepare tiny scales fused={fused}")
    M, K = (2, 512) if fused else (4, 512)
    x = S.activations(M, K, seed=5, n_outliers=2)
    x[1] *= np.float32(1e-33)                          # amax ~ 1e-32: s_x < 2^-100
    if M > 2:
        x[2] = np.float32(1e-40) * np.sign(x[2])       # subnormal inputs
        x[3] *= np.float32(3e-29)                      # just above the fast-path limit
    xq_ref, sx_ref = O.prepare(x)
    if fused:
        _, q = oracle_layer(64, K, 1)
        L = gpu_layer(w, q)
        x_q = torch.empty((M, K), dtype=torch.int8, device=DEV)
        s_x = torch.empty((M,), dtype=torch.float32, device=DEV)
        w.forward(gpu(x), L, x_q=x_q, s_x=s_x)
        xq, sx = x_q, s_x
    else:
        xq, sx = w.prepare_activation(gpu(x))
    torch.cuda.synchronize()
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


# ----------------------------------------------------------------------------- quantize

def check_quant(w, W, seed, dtype=torch.float32):
    q = O.quantize_weight(W, seed=seed)
    Wg = gpu(W) if dtype == torch.float32 else gpu(S.to_bf16_bits(W).view(np.int16)).view(torch.bfloat16)
    L = w.quantize_weight(Wg, seed=seed)
    torch.cuda.synchronize()
    assert np.array_equal(L.codebook.cpu().numpy().view(np.uint32), q["cb"].view(np.uint32))
    assert np.array_equal(L.s_channel.cpu().numpy().view(np.uint32), q["s_ch"].view(np.uint32))
    assert np.array_equal(L.s_rel.cpu().numpy(), q["s_rel"])
    assert np.array_equal(L.packed.cpu().numpy(), q["packed"])
    return L, q


# rows of 1 to 128 blocks take the row-transform scale kernel (one or two rounds), longer
# rows the lane-transform one; 40 x 33024 also samples (over 2^20 values)
@pytest.mark.parametrize("N,K,seed", [(256, 512, 0), (1, 256, 3), (2048, 1024, 42), (300, 768, 7),
                                      (64, 32768, 11), (40, 33024, 5)])
def test_quantize_bit_exact(w, N, K, seed):
    say(f"quantize N={N} K={K} seed={seed}")
    W = S.weights(N, K, seed=seed)
    check_quant(w, W, seed)


def test_quantize_zero_rows_and_blocks(w):
    # exact zeros of both signs: a zero row, a -0 row, a zero block and a -0 block (the row
    # transform may give -0 where the lane transform gives +0; no output may show it)
    say("quantize zero rows and blocks")
    W = S.weights(64, 1024, seed=13)
    W[3] = 0.0
    W[5] = -0.0
    W[7, 256:512] = 0.0
    W[9, 512:768] = -0.0
    check_quant(w, W, 13)


def test_quantize_bf16_input(w):
    say("quantize bf16 N=64 K=768")
    W = S.bf16_bits_to_f32(S.to_bf16_bits(S.weights(64, 768, seed=5)))
    check_quant(w, W, 5, dtype=torch.bfloat16)


def test_quantize_constructed_layer_exact(w):
    from test_oracle import constructed_layer
    say("quantize constructed layer")
    W, truth = constructed_layer()
    L, _ = check_quant(w, W, 0)
    assert np.array_equal(L.packed.cpu().numpy(), truth["packed"])
    assert np.array_equal(L.codebook.cpu().numpy(), truth["cb"])


@pytest.mark.parametrize("N,K", [S.MLP_GATE_UP, S.MLP_DOWN])
def test_quantize_full_size(w, N, K):
    say(f"quantize full N={N} K={K}")
    W, q = oracle_layer(N, K)
    L = w.quantize_weight(gpu(W), seed=0)
    torch.cuda.synchronize()
    assert np.array_equal(L.codebook.cpu().numpy().view(np.uint32), q["cb"].view(np.uint32))
    assert np.array_equal(L.s_channel.cpu().numpy().view(np.uint32), q["s_ch"].view(np.uint32))
    assert np.array_equal(L.s_rel.cpu().numpy(), q["s_rel"])
    assert np.array_equal(L.packed.cpu().numpy(), q["packed"])


def test_quantize_two_sampling_passes(w):
    # more 256-blocks than one pass of the sampler's per-block buckets covers (2^19 - 1024
    # blocks), so the fit sample is gathered in two passes over block ranges
    N, K = 33280, 4096
    say(f"quantize two sampling passes N={N} K={K}")
    W = np.random.default_rng(7).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    q = O.quantize_weight(W, seed=3)
    L = w.quantize_weight(gpu(W), seed=3)
    torch.cuda.synchronize()
    assert np.array_equal(L.codebook.cpu().numpy().view(np.uint32), q["cb"].view(np.uint32))
    assert np.array_equal(L.s_rel.cpu().numpy(), q["s_rel"])
    assert np.array_equal(L.packed.cpu().numpy(), q["packed"])


# ----------------------------------------------------------------------------- linear

def run_linear(w, algo, N, K, M, rows=None, toks=None, out_dtype=torch.float32, seed=0, n_out=None):
    _, q = oracle_layer(N, K, seed)
    _, xq, sx = oracle_acts(M, K, seed, n_out)
    L = gpu_layer(w, q)
    y = w.linear(gpu(xq), gpu(sx), L, out_dtype=out_dtype, algo=algo)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    if rows is not None or toks is not None:
        rr = np.arange(N) if rows is None else rows
        tt = np.arange(M) if toks is None else toks
        y = y[np.ix_(tt, rr)]
    yr, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, toks)
    return y, yr, A, (q, xq, sx)


def assert_gate(y, yr, A, extra=0.0):
    err = np.abs(y - yr)
    bound = 4e-3 * A + extra
    zero = A == 0
    assert np.all(y[zero] == 0)
    ratio = err[~zero] / bound[~zero]
    say(f"  max |y - y_ref| / (4e-3 A) = {ratio.max():.4f}")
    assert np.all(err <= bound)


GEMV_CASES = [(256, 512, 1), (256, 512, 2), (256, 512, 3), (256, 512, 4), (1001, 768, 3), (1, 256, 1),
              (8, 10240, 4)]


@pytest.mark.parametrize("N,K,M", GEMV_CASES)
def test_gemv_parity(w, N, K, M):
    say(f"gemv N={N} K={K} M={M}")
    y, yr, A, _ = run_linear(w, w.ALGO_GEMV, N, K, M, n_out=2)
    assert_gate(y, yr, A)


@pytest.mark.parametrize("N,K,M", [(17408, 5120, 1), (5120, 17408, 1), (17408, 5120, 2), (5120, 17408, 2)])
def test_gemv_full_size_sampled(w, N, K, M):
    say(f"gemv full N={N} K={K} M={M}")
    rows = sample(N, 2048, N + M)
    y, yr, A, _ = run_linear(w, w.ALGO_GEMV, N, K, M, rows=rows)
    assert_gate(y, yr, A)


def i8_tight(y, q, xq, sx, rows, toks):
    y8, A8 = O.linear_i8_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, toks)
    G = xq.shape[1] // 16
    err = np.abs(y - y8)
    bound = (G + 4) * U32 * A8
    say(f"  max |y - y8| / ((G+4) u A8) = {np.max(err / np.maximum(bound, 1e-300)):.4f}")
    assert np.all(err <= bound)


# 256-token x 192-row tiles: ragged in both directions, several tiles each way, K = 256 (one
# turn of the four-stage ring)
# the two int8-codebook kernels: the group scale inside the fp16 weight, and the int8 MFMA
# with the per-group fold on the vector ALU
I8_ALGOS = {"mfma_i8": 2, "mfma_i8_fold": 6}


@pytest.mark.parametrize("algo", list(I8_ALGOS))
@pytest.mark.parametrize("N,K,M", [(256, 512, 4), (200, 768, 37), (300, 1024, 130), (128, 256, 128),
                                   (385, 1280, 600), (193, 256, 65), (1000, 2048, 513)])
def test_mfma_i8_parity(w, N, K, M, algo):
    say(f"{algo} N={N} K={K} M={M}")
    y, yr, A, (q, xq, sx) = run_linear(w, I8_ALGOS[algo], N, K, M, n_out=2)
    assert_gate(y, yr, A)
    i8_tight(y, q, xq, sx, None, None)


@pytest.mark.parametrize("algo", list(I8_ALGOS))
@pytest.mark.parametrize("N,K", [S.MLP_GATE_UP, S.MLP_DOWN])
def test_mfma_i8_full_size_sampled(w, N, K, algo):
    M = 2048
    say(f"{algo} full N={N} K={K} M={M}")
    rows, toks = sample(N, 384, N), sample(M, 48, M + 1)
    y, yr, A, (q, xq, sx) = run_linear(w, I8_ALGOS[algo], N, K, M, rows=rows, toks=toks)
    assert_gate(y, yr, A)
    i8_tight(y, q, xq, sx, rows, toks)


# 256-token x 192-row tiles: ragged in both directions, several tiles each way, K = 256 (one
# turn of the four-stage ring)
@pytest.mark.parametrize("N,K,M", [(256, 512, 4), (200, 768, 37), (300, 1024, 130), (512, 256, 257),
                                   (17, 5120, 3), (385, 1280, 600), (193, 256, 65), (1000, 2048, 513)])
def test_mfma_f16_parity(w, N, K, M):
    say(f"mfma_f16 N={N} K={K} M={M}")
    y, yr, A, _ = run_linear(w, w.ALGO_MFMA_F16, N, K, M, n_out=2)
    assert_gate(y, yr, A)


@pytest.mark.parametrize("N,K", [S.MLP_GATE_UP, S.MLP_DOWN])
def test_mfma_f16_full_size_sampled(w, N, K):
    M = 2048
    say(f"mfma_f16 full N={N} K={K} M={M}")
    rows, toks = sample(N, 384, N), sample(M, 48, M + 1)
    y, yr, A, _ = run_linear(w, w.ALGO_MFMA_F16, N, K, M, rows=rows, toks=toks)
    assert_gate(y, yr, A)


@pytest.mark.parametrize("algo", ["mfma_i8", "mfma_i8_fold", "mfma_f16"])
def test_prefill_longest_rows(w, algo):
    """K = 131072 (512 rotation blocks, 8192 groups per row) through the two decoded-weight
    prefill routes: random layer bytes in the format's ranges, sampled rows and tokens against
    the oracle's product (and, for the int8 route, its int8-codebook reading)."""
    N, K, M = 200, 131072, 300
    a = {"mfma_i8": w.ALGO_MFMA_I8, "mfma_i8_fold": w.ALGO_MFMA_I8_FOLD, "mfma_f16": w.ALGO_MFMA_F16}[algo]
    say(f"{algo} longest rows N={N} K={K} M={M}")
    g = np.random.default_rng(12)
    packed = g.integers(-128, 128, size=(N, K // 2), dtype=np.int8)
    s_rel = g.integers(0x20, 0x39, size=(N, K // 16), dtype=np.uint8)
    s_ch = (0.01 + 0.02 * g.random(N)).astype(np.float32)
    cb = np.sort(g.standard_normal(16)).astype(np.float32)
    _, xq, sx = oracle_acts(M, K, 13, 2)
    L = w.QuantizedLinear(gpu(packed), gpu(s_rel), gpu(s_ch), gpu(cb))
    y = w.linear(gpu(xq), gpu(sx), L, algo=a)
    torch.cuda.synchronize()
    rows, toks = sample(N, 24, 7), sample(M, 24, 8)
    y = y.cpu().numpy().astype(np.float64)[np.ix_(toks, rows)]
    yr, A = O.linear_ref(xq, sx, packed, s_rel, s_ch, cb, rows, toks)
    assert_gate(y, yr, A)
    if algo.startswith("mfma_i8"):
        i8_tight(y, {"packed": packed, "s_rel": s_rel, "s_ch": s_ch, "cb": cb}, xq, sx, rows, toks)


# Requantised int8 weights: the kernel and the oracle take the same integer decisions (the
# table of rounded group-scaled levels, exact int32 sums) and the same three fp32 roundings,
# so the outputs are compared bit for bit; the gate against the exact product is the
# tolerance study of this reading.
def run_rq(w, N, K, M, rows=None, toks=None, out_dtype=torch.float32, seed=0, layer=None):
    if layer is None:
        _, q = oracle_layer(N, K, seed)
        layer = (q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    _, xq, sx = oracle_acts(M, K, seed, 2)
    L = w.QuantizedLinear(*(gpu(t) for t in layer))
    y = w.linear(gpu(xq), gpu(sx), L, out_dtype=out_dtype, algo=w.ALGO_MFMA_RQ)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    rr = np.arange(N) if rows is None else rows
    tt = np.arange(M) if toks is None else toks
    y = y[np.ix_(tt, rr)]
    yq = O.linear_rq_ref(xq, sx, *layer, rows, toks)
    return y, yq, (xq, sx, layer)


@pytest.mark.parametrize("N,K,M", [(256, 512, 4), (200, 768, 37), (300, 1024, 130), (512, 256, 257),
                                   (17, 5120, 3), (385, 1280, 600), (193, 256, 65), (1000, 2048, 513),
                                   (1, 256, 1)])
def test_mfma_rq_parity(w, N, K, M):
    say(f"mfma_rq N={N} K={K} M={M}")
    y, yq, (xq, sx, layer) = run_rq(w, N, K, M)
    assert np.array_equal(y.view(np.uint32), yq.view(np.uint32))
    yr, A = O.linear_ref(xq, sx, *layer)
    assert_gate(y.astype(np.float64), yr, A)


@pytest.mark.parametrize("N,K", [S.MLP_GATE_UP, S.MLP_DOWN])
def test_mfma_rq_full_size_sampled(w, N, K):
    M = 2048
    say(f"mfma_rq full N={N} K={K} M={M}")
    rows, toks = sample(N, 384, N), sample(M, 48, M + 1)
    y, yq, (xq, sx, layer) = run_rq(w, N, K, M, rows=rows, toks=toks)
    assert np.array_equal(y.view(np.uint32), yq.view(np.uint32))
    yr, A = O.linear_ref(xq, sx, *layer, rows, toks)
    assert_gate(y.astype(np.float64), yr, A)


def test_mfma_rq_every_scale_code(w):
    """Random layer bytes with group-scale codes over the whole e4m3 range, the NaN codes and
    scales above 1 (whose levels clamp at +-127) included: the clamping and NaN rules of the
    table, bit for bit."""
    N, K, M = 300, 1024, 70
    g = np.random.default_rng(8)
    packed = g.integers(-128, 128, size=(N, K // 2), dtype=np.int8)
    s_rel = g.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    s_ch = (0.01 + 0.02 * g.random(N)).astype(np.float32)
    cb = np.sort(g.standard_normal(16)).astype(np.float32)
    say(f"mfma_rq all codes N={N} K={K} M={M}")
    y, yq, _ = run_rq(w, N, K, M, layer=(packed, s_rel, s_ch, cb))
    assert np.array_equal(y.view(np.uint32), yq.view(np.uint32))


def test_mfma_rq_longest_rows_extreme_values(w):
    """K = 131072, the longest rows the route takes, with every product at +-127 x 127: the
    int32 sums reach 127^2 K = 2.11e9, just under 2^31, and must stay exact.  Rows alternate
    the sign of their level; sampled rows and tokens against the oracle, bit for bit."""
    N, K, M = 200, 131072, 300
    say(f"mfma_rq extreme N={N} K={K} M={M}")
    cb = np.linspace(-1.0, 1.0, 16).astype(np.float32)        # levels 0 and 15 map to -127 / +127
    packed = np.full((N, K // 2), -1, dtype=np.int8)           # index 15 in both nibbles
    packed[1::2] = 0                                           # index 0
    s_rel = np.full((N, K // 16), 0x38, dtype=np.uint8)        # 1.0
    s_ch = np.full(N, 0.5, dtype=np.float32)
    xq = np.full((M, K), 127, dtype=np.int8)
    xq[::3] = -127
    sx = np.full(M, 0.25, dtype=np.float32)
    L = w.QuantizedLinear(gpu(packed), gpu(s_rel), gpu(s_ch), gpu(cb))
    y = w.linear(gpu(xq), gpu(sx), L, algo=w.ALGO_MFMA_RQ)
    torch.cuda.synchronize()
    rows, toks = sample(N, 24, 3), sample(M, 24, 4)
    y = y.cpu().numpy()[np.ix_(toks, rows)]
    yq = O.linear_rq_ref(xq, sx, packed, s_rel, s_ch, cb, rows, toks)
    assert np.array_equal(y.view(np.uint32), yq.view(np.uint32))
    t = O.rq_table(cb)
    assert t[0x38, 15] == 127 and t[0x38, 0] == -127
    sw = np.float32(0.5) * (np.float32(1.0) / np.float32(127.0))   # s_channel * s_cb
    assert np.abs(yq).max() == (np.float32(127 * 127 * K) * sw) * np.float32(0.25)


def test_mfma_rq_bf16_output(w):
    N, K, M = 385, 768, 300
    say(f"mfma_rq bf16 N={N} K={K} M={M}")
    y, yq, _ = run_rq(w, N, K, M, out_dtype=torch.bfloat16)
    want = torch.from_numpy(yq).to(torch.bfloat16).float().numpy()   # round to nearest even
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))


# (N, K, M): 16-row tiles per workgroup 1..5 (N = 2048, 5120, 10000, 15360, 17408 on 256 CUs),
# token tiles 1..4, ragged N and M, K = 256 (waves with no K range)
SKINNY_CASES = [(256, 512, 3), (300, 768, 17), (1001, 1024, 33), (17, 5120, 64), (64, 256, 5),
                (2048, 1280, 48), (5120, 768, 16), (10000, 256, 40), (15360, 256, 2), (17408, 256, 8)]


@pytest.mark.parametrize("N,K,M", SKINNY_CASES)
def test_mfma_skinny_parity(w, N, K, M):
    say(f"mfma_skinny N={N} K={K} M={M}")
    y, yr, A, _ = run_linear(w, w.ALGO_MFMA_SKINNY, N, K, M, n_out=2)
    assert_gate(y, yr, A)


@pytest.mark.parametrize("N,K,M", [(17408, 5120, 64), (5120, 17408, 16), (15360, 5120, 33), (5120, 5120, 64)])
def test_mfma_skinny_full_size_sampled(w, N, K, M):
    say(f"mfma_skinny full N={N} K={K} M={M}")
    rows = sample(N, 512, N + M)
    y, yr, A, _ = run_linear(w, w.ALGO_MFMA_SKINNY, N, K, M, rows=rows)
    assert_gate(y, yr, A)


# shapes whose batched decode splits K in 4 on a 256-CU device (more than 16 tokens, K a
# multiple of 1024 of at least 8192, few rows per CU), ragged row blocks and token tiles
# included
SPLIT_CASES = [(1000, 8192, 24, 4), (300, 8192, 40, 4), (5120, 8192, 17, 4), (77, 8192, 64, 4)]


def run_linear_ws(w, N, K, M, rows=None, out_dtype=torch.float32, seed=0, n_out=None, ws=None):
    _, q = oracle_layer(N, K, seed)
    _, xq, sx = oracle_acts(M, K, seed, n_out)
    L = gpu_layer(w, q)
    if ws is None:
        ws = w.linear_workspace(M, N, K)
    y = w.linear_ws(gpu(xq), gpu(sx), L, ws, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        y = y[:, rows]
    yr, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows)
    return y, yr, A, ws


def counters_clear(ws, M, N, parts):
    """The arrival counters (the workspace's first 4 KiB, before the parts' sums) are all back
    to zero."""
    assert ws.numel() == 4096 + parts * M * N * 4
    return int(ws[:4096].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("N,K,M,parts", SPLIT_CASES)
def test_mfma_skinny_split_parity(w, N, K, M, parts):
    """The batched decode with K split across workgroups (w4a8_linear_ws): within the gate,
    the workspace's counters back at zero, two calls in a row (the second on a smaller
    input sharing the workspace) and a repeat bit-identical."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if ncu != 256:
        pytest.skip(f"split shapes chosen for 256 compute units, this device has {ncu}")
    say(f"mfma_skinny split N={N} K={K} M={M} parts={parts}")
    nb = w.linear_workspace_bytes(M, N, K)
    assert nb == 4096 + parts * M * N * 4
    y, yr, A, ws = run_linear_ws(w, N, K, M, n_out=2)
    assert_gate(y, yr, A)
    assert counters_clear(ws, M, N, parts)
    y2, yr2, A2, _ = run_linear_ws(w, N, K, max(4, M // 2), seed=1, ws=ws)
    assert_gate(y2, yr2, A2)
    y3, _, _, _ = run_linear_ws(w, N, K, M, n_out=2, ws=ws)
    assert np.array_equal(y, y3)
    assert counters_clear(ws, M, N, parts)


def test_mfma_skinny_split_full_size_and_fallback(w):
    """The MLP down projection at 64 tokens splits K in 4; bf16 output; with no workspace (or
    one too small) linear_ws runs as linear does, bit for bit."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if ncu != 256:
        pytest.skip(f"split shapes chosen for 256 compute units, this device has {ncu}")
    N, K, M = 5120, 17408, 64
    say(f"mfma_skinny split full N={N} K={K} M={M}")
    rows = sample(N, 512, N + M)
    y, yr, A, ws = run_linear_ws(w, N, K, M, rows=rows)
    assert_gate(y, yr, A)
    yb, yrb, Ab, _ = run_linear_ws(w, N, K, M, rows=rows, out_dtype=torch.bfloat16, ws=ws)
    assert_gate(yb, yrb, Ab, extra=2.0 ** -8 * np.abs(yrb))
    assert counters_clear(ws, M, N, 4)
    y0, _, _, _ = run_linear_ws(w, N, K, M, rows=rows, ws=torch.zeros(0, dtype=torch.uint8, device="cuda"))
    y1, _, _, _ = run_linear(w, w.ALGO_AUTO, N, K, M, rows=rows)
    assert np.array_equal(y0, y1)


def test_mfma_skinny_long_rows(w):
    """Rows so long that a workgroup's staged group scales leave room for fewer row tiles
    (12304 x 32768 wants four 16-row tiles per workgroup; three fit beside the table).  The
    layer is made of random bytes in the format's ranges rather than quantised (the product
    is defined by the four tensors alone); sampled rows against the oracle's product."""
    N, K, M = 12304, 32768, 8
    say(f"mfma_skinny long rows N={N} K={K} M={M}")
    g = np.random.default_rng(5)
    packed = g.integers(-128, 128, size=(N, K // 2), dtype=np.int8)
    s_rel = g.integers(0x20, 0x39, size=(N, K // 16), dtype=np.uint8)  # e4m3 codes in [2^-4, 1]
    s_ch = (0.01 + 0.02 * g.random(N)).astype(np.float32)
    cb = np.sort(g.standard_normal(16)).astype(np.float32)
    _, xq, sx = oracle_acts(M, K, 9, 2)
    L = w.QuantizedLinear(gpu(packed), gpu(s_rel), gpu(s_ch), gpu(cb))
    y = w.linear(gpu(xq), gpu(sx), L, algo=w.ALGO_MFMA_SKINNY)
    torch.cuda.synchronize()
    rows = sample(N, 256, 11)
    y = y.float().cpu().numpy().astype(np.float64)[:, rows]
    yr, A = O.linear_ref(xq, sx, packed, s_rel, s_ch, cb, rows, None)
    assert_gate(y, yr, A)


@pytest.mark.parametrize("algo", ["gemv", "mfma_i8", "mfma_f16", "mfma_skinny", "mfma_i8_fold"])
def test_bf16_output(w, algo):
    a = {"gemv": 1, "mfma_i8": 2, "mfma_f16": 3, "mfma_skinny": 4, "mfma_i8_fold": 6}[algo]
    say(f"bf16 output {algo}")
    y, yr, A, _ = run_linear(w, a, 256, 512, 2, out_dtype=torch.bfloat16, n_out=2)
    assert_gate(y, yr, A, extra=2.0 ** -8 * np.abs(yr))


@pytest.mark.parametrize("algo,M", [(1, 1), (1, 4), (2, 64), (3, 64), (4, 3), (4, 64), (5, 300), (6, 300),
                                    (0, 1), (0, 8), (0, 300)])
def test_deterministic_and_auto(w, algo, M):
    say(f"determinism algo={algo} M={M}")
    N, K = 512, 1024
    _, q = oracle_layer(N, K)
    _, xq, sx = oracle_acts(M, K)
    L = gpu_layer(w, q)
    xg, sg = gpu(xq), gpu(sx)
    a = w.linear(xg, sg, L, algo=algo)
    b = w.linear(xg, sg, L, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    yr, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    assert_gate(a.cpu().numpy().astype(np.float64), yr, A)


def test_end_to_end_layer_call(w):
    say("end-to-end layer call")
    N, K, M = 512, 768, 3
    W = S.weights(N, K, seed=11)
    x = S.activations(M, K, seed=11, n_outliers=2)
    L = w.quantize_weight(gpu(W), seed=11)
    y = L(gpu(x))
    torch.cuda.synchronize()
    q = O.quantize_weight(W, seed=11)
    xq, sx = O.prepare(x)
    yr, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    assert_gate(y.cpu().numpy().astype(np.float64), yr, A)


# fused (M = 1, K <= 32768; M = 2, K <= 20480) and two-launch cases on both sides of each limit
FWD_CASES = [(256, 512, 1, "f32"), (256, 512, 2, "bf16"), (1001, 768, 1, "bf16"), (64, 20480, 1, "f32"),
             (8, 20480, 2, "f32"), (300, 256, 2, "f32"), (200, 1024, 7, "f32"), (128, 20736, 1, "bf16"),
             (64, 32768, 1, "bf16"), (40, 33024, 1, "f32"), (24, 20736, 2, "f32")]


@pytest.mark.parametrize("N,K,M,dt", FWD_CASES)
def test_forward_fused_and_fallback(w, N, K, M, dt):
    """w4a8_forward: x_q and s_x bit-exact with the oracle's preparation, y within the bound
    (one launch for M = 1, K <= 32768 and M = 2, K <= 20480; two launches otherwise)."""
    say(f"forward N={N} K={K} M={M} {dt}")
    _, q = oracle_layer(N, K, 3)
    x = S.activations(M, K, seed=N + K + M, n_outliers=2)
    if M > 1:
        x[1] = 0.0  # an all-zero token
    if dt == "bf16":
        bits = S.to_bf16_bits(x)
        xin = gpu(bits.view(np.int16)).view(torch.bfloat16)
        x = S.bf16_bits_to_f32(bits)
    else:
        xin = gpu(x)
    xq_ref, sx_ref = O.prepare(x)
    L = gpu_layer(w, q)
    x_q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s_x = torch.empty((M,), dtype=torch.float32, device=DEV)
    y = w.forward(xin, L, x_q=x_q, s_x=s_x)
    torch.cuda.synchronize()
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(x_q.cpu().numpy(), xq_ref)
    yr, A = O.linear_ref(xq_ref, sx_ref, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    assert_gate(y.cpu().numpy().astype(np.float64), yr, A)


def test_safetensors_round_trip_on_gpu(w, tmp_path):
    """Quantise on the GPU, write the four tensors, read them back onto the GPU: the layer's
    output is bit-identical to the original's."""
    from w4a8_codebook_gemm_amd import safetensors_io as io
    say("safetensors round trip on the GPU")
    W = gpu(S.weights(300, 1024, seed=9))
    L = w.quantize_weight(W, seed=9)
    path = str(tmp_path / "layer.safetensors")
    io.save_layers(path, {"model.layers.3.mlp.up_proj": L})
    L2 = io.load_layers(path, device=DEV)["model.layers.3.mlp.up_proj"]
    x = gpu(S.activations(2, 1024, seed=9))
    y1, y2 = w.forward(x, L), w.forward(x, L2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ----------------------------------------------------------------------------- scale codes

def random_layer(N, K, seed, codes):
    """Layer bytes drawn uniformly: packed indices, group-scale bytes from `codes`, row scales
    in [0.01, 0.03], a sorted normal codebook (the product is defined by the four tensors)."""
    g = np.random.default_rng(seed)
    packed = g.integers(-128, 128, size=(N, K // 2), dtype=np.int8)
    s_rel = g.choice(np.asarray(codes, dtype=np.uint8), size=(N, K // 16))
    s_ch = (0.01 + 0.02 * g.random(N)).astype(np.float32)
    cb = np.sort(g.standard_normal(16)).astype(np.float32)
    return packed, s_rel, s_ch, cb


# every e4m3 code but the two NaN codes: subnormal scales 0x01-0x07 (which the quantiser
# writes for groups under 2^-6 of the row maximum), scales above 1 up to 448 (0x39-0x7E,
# which the format's relative scale never reaches but a producer may write), and negative
# codes 0x80-0xFE
ALL_FINITE_CODES = [c for c in range(256) if c not in (0x7F, 0xFF)]


@pytest.mark.parametrize("algo,N,K,M", [("gemv", 300, 1024, 1), ("gemv", 257, 2048, 3),
                                        ("mfma_skinny", 300, 1024, 8), ("mfma_skinny", 1001, 768, 64),
                                        ("mfma_i8", 300, 1024, 300), ("mfma_f16", 300, 1024, 300),
                                        ("mfma_i8", 200, 768, 8), ("mfma_f16", 200, 768, 8),
                                        ("mfma_i8_fold", 300, 1024, 300)])
def test_every_scale_code(w, algo, N, K, M):
    """Random group-scale bytes over every finite E4M3FN code (each appears over a hundred
    times) through each kernel that decodes them with the hardware conversion, against the
    oracle's exact product; the int8 route also against its int8-codebook reading."""
    a = {"gemv": w.ALGO_GEMV, "mfma_skinny": w.ALGO_MFMA_SKINNY, "mfma_i8": w.ALGO_MFMA_I8,
         "mfma_f16": w.ALGO_MFMA_F16, "mfma_i8_fold": w.ALGO_MFMA_I8_FOLD}[algo]
    say(f"{algo} every scale code N={N} K={K} M={M}")
    packed, s_rel, s_ch, cb = random_layer(N, K, 21 + M, ALL_FINITE_CODES)
    assert len(np.unique(s_rel)) == len(ALL_FINITE_CODES)
    _, xq, sx = oracle_acts(M, K, 31, 2)
    L = w.QuantizedLinear(gpu(packed), gpu(s_rel), gpu(s_ch), gpu(cb))
    y = w.linear(gpu(xq), gpu(sx), L, algo=a)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    yr, A = O.linear_ref(xq, sx, packed, s_rel, s_ch, cb)
    assert_gate(y, yr, A)
    if algo.startswith("mfma_i8"):
        i8_tight(y, {"packed": packed, "s_rel": s_rel, "s_ch": s_ch, "cb": cb}, xq, sx, None, None)


@pytest.mark.parametrize("algo,M", [("gemv", 1), ("mfma_skinny", 8), ("mfma_skinny", 40), ("mfma_i8", 300),
                                    ("mfma_f16", 300), ("mfma_i8_fold", 300)])
def test_every_scale_code_per_row(w, algo, M):
    """Row r's group scales are all the r-th finite E4M3FN code, so each output row sees one
    decoded scale alone: a code decoded wrongly (a subnormal flushed to zero, a sign or an
    exponent off) moves that row's outputs far outside the per-output gate, which a mix of
    codes within a row could hide behind its larger groups."""
    a = {"gemv": w.ALGO_GEMV, "mfma_skinny": w.ALGO_MFMA_SKINNY, "mfma_i8": w.ALGO_MFMA_I8,
         "mfma_f16": w.ALGO_MFMA_F16, "mfma_i8_fold": w.ALGO_MFMA_I8_FOLD}[algo]
    N, K = 300, 1024
    say(f"{algo} one scale code per row N={N} K={K} M={M}")
    packed, s_rel, s_ch, cb = random_layer(N, K, 41 + M, ALL_FINITE_CODES)
    s_rel[:len(ALL_FINITE_CODES)] = np.asarray(ALL_FINITE_CODES, dtype=np.uint8)[:, None]
    _, xq, sx = oracle_acts(M, K, 43, 2)
    L = w.QuantizedLinear(gpu(packed), gpu(s_rel), gpu(s_ch), gpu(cb))
    y = w.linear(gpu(xq), gpu(sx), L, algo=a)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    yr, A = O.linear_ref(xq, sx, packed, s_rel, s_ch, cb)
    nonzero = [r for r, c in enumerate(ALL_FINITE_CODES) if c & 0x7F]  # 0x00 and 0x80 decode to zero
    assert np.all(np.abs(yr[:, nonzero]) > 0)
    assert_gate(y, yr, A)
    if algo.startswith("mfma_i8"):
        i8_tight(y, {"packed": packed, "s_rel": s_rel, "s_ch": s_ch, "cb": cb}, xq, sx, None, None)


# ----------------------------------------------------------------------------- benchmarked launches

def test_bench_gate_up_launch_full_size(w):
    """The benchmark's dominant launch as it runs there: w4a8_forward_multi over gate and up
    (two 17408 x 5120 layers, one launch), fp32 activations of one token with 0.1% outlier
    channels.  x_q and s_x bit-exact; 2048 sampled rows of each layer within the bound."""
    (N, K) = S.MLP_GATE_UP
    say(f"bench launch: forward_multi gate+up 2 x {N}x{K}, M=1, fp32 x")
    qs = [oracle_layer(N, K, 0)[1], oracle_layer(N, K, 1)[1]]
    x = S.activations(1, K, seed=0)
    xq_ref, sx_ref = O.prepare(x)
    Ls = [gpu_layer(w, q) for q in qs]
    x_q = torch.empty((1, K), dtype=torch.int8, device=DEV)
    s_x = torch.empty((1,), dtype=torch.float32, device=DEV)
    ys = w.forward_multi(gpu(x), Ls, x_q=x_q, s_x=s_x)
    torch.cuda.synchronize()
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(x_q.cpu().numpy(), xq_ref)
    for g, q in enumerate(qs):
        rows = sample(N, 2048, 100 + g)
        y = ys[g].cpu().numpy().astype(np.float64)[:, rows]
        yr, A = O.linear_ref(xq_ref, sx_ref, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, None)
        assert_gate(y, yr, A)


def test_bench_down_launch_full_size(w):
    """The benchmark's second launch: w4a8_forward over down (5120 x 17408), fp32
    activations of one token; x_q and s_x bit-exact, 2048 sampled rows within the bound."""
    (N, K) = S.MLP_DOWN
    say(f"bench launch: forward down {N}x{K}, M=1, fp32 x")
    _, q = oracle_layer(N, K, 0)
    x = S.activations(1, K, seed=1)
    xq_ref, sx_ref = O.prepare(x)
    x_q = torch.empty((1, K), dtype=torch.int8, device=DEV)
    s_x = torch.empty((1,), dtype=torch.float32, device=DEV)
    y = w.forward(gpu(x), gpu_layer(w, q), x_q=x_q, s_x=s_x)
    torch.cuda.synchronize()
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(x_q.cpu().numpy(), xq_ref)
    rows = sample(N, 2048, 102)
    yr, A = O.linear_ref(xq_ref, sx_ref, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, None)
    assert_gate(y.cpu().numpy().astype(np.float64)[:, rows], yr, A)



def test_bench_model_attention_launches_full_size(w):
    """The 62-layer decoder's attention launches as the benchmark runs them: w4a8_forward_multi
    over four 5120 x 5120 layers (one launch) and w4a8_forward over a fifth, fp32 activations
    of one token.  The five layers come from one oracle quantisation, rows permuted (r -> p r
    mod N for odd p prime to 5) and row scales multiplied by g + 1, so each layer is distinct
    and a launch that mixed them up would fail.  x_q and s_x bit-exact; 1024 sampled rows of
    each layer within the bound."""
    (N, K) = S.ATTN_SQUARE
    say(f"bench launch: forward_multi 4 x {N}x{K} and forward {N}x{K}, M=1, fp32 x")
    _, q0 = oracle_layer(N, K, 0)
    qs = []
    for g, p in enumerate((1, 3, 7, 11, 13)):
        perm = (np.arange(N) * p) % N
        qs.append(dict(packed=q0["packed"][perm], s_rel=q0["s_rel"][perm],
                       s_ch=(q0["s_ch"][perm] * np.float32(g + 1)).astype(np.float32), cb=q0["cb"]))
    for qset, seed in ((qs[:4], 3), (qs[4:], 4)):
        x = S.activations(1, K, seed=seed)
        xq_ref, sx_ref = O.prepare(x)
        Ls = [gpu_layer(w, q) for q in qset]
        x_q = torch.empty((1, K), dtype=torch.int8, device=DEV)
        s_x = torch.empty((1,), dtype=torch.float32, device=DEV)
        if len(Ls) > 1:
            ys = w.forward_multi(gpu(x), Ls, x_q=x_q, s_x=s_x)
        else:
            ys = [w.forward(gpu(x), Ls[0], x_q=x_q, s_x=s_x)]
        torch.cuda.synchronize()
        assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
        assert np.array_equal(x_q.cpu().numpy(), xq_ref)
        for g, q in enumerate(qset):
            rows = sample(N, 1024, 200 + g)
            yr, A = O.linear_ref(xq_ref, sx_ref, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, None)
            assert_gate(ys[g].cpu().numpy().astype(np.float64)[:, rows], yr, A)


# ----------------------------------------------------------------------------- binding checks

def test_binding_refuses_wrong_buffers(w):
    """Caller-supplied outputs of the wrong shape are refused before anything is launched
    (the C ABI cannot see buffer sizes), and the outputs keep their contents."""
    say("binding refuses undersized and misshapen buffers")
    N, K, M = 256, 512, 4
    _, q = oracle_layer(N, K)
    _, xq, sx = oracle_acts(M, K)
    L = gpu_layer(w, q)
    xg, sg = gpu(xq), gpu(sx)
    x = gpu(S.activations(M, K, seed=3))
    short_y = torch.full((M, N - 1), 7.0, device=DEV)
    with pytest.raises(ValueError):
        w.linear(xg, sg, L, out=short_y)
    with pytest.raises(ValueError):
        w.linear(xg, sg, L, out=torch.empty((N, M), device=DEV))
    with pytest.raises(ValueError):
        w.forward(x, L, out=short_y)
    with pytest.raises(ValueError):
        w.forward(x, L, x_q=torch.empty((M, K - 16), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):
        w.forward(x, L, s_x=torch.empty((M - 1,), device=DEV))
    with pytest.raises(ValueError):
        w.prepare_activation(x, out=(torch.empty((M, K // 2), dtype=torch.int8, device=DEV),
                                     torch.empty((M,), device=DEV)))
    with pytest.raises(ValueError):
        w.prepare_activation(x, out=(torch.empty((M, K), dtype=torch.int8, device=DEV),
                                     torch.empty((M + 1,), device=DEV)))
    with pytest.raises(ValueError):
        w.linear_multi(xg, sg, [L, L], outs=[torch.empty((M, N), device=DEV), short_y])
    with pytest.raises(ValueError):
        w.forward_multi(x, [L, L], outs=[short_y, torch.empty((M, N), device=DEV)])
    with pytest.raises(ValueError):
        w.forward_multi(x, [L], x_q=torch.empty((1, K), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):   # a layer tensor of the wrong length
        w.linear(xg, sg, w.QuantizedLinear(L.packed, L.s_rel, L.s_channel[:-1], L.codebook))
    W8 = w.w8a8_quantize_weight(gpu(S.weights(N, K, seed=1)))
    with pytest.raises(ValueError):
        w.w8a8_linear(xg, sg, W8, out=short_y)
    x_cpu = torch.empty((M, K), dtype=torch.int8)
    with pytest.raises(ValueError):
        w.linear(x_cpu, sg, L)
    torch.cuda.synchronize()
    assert torch.all(short_y == 7.0)
