"""Parity of the W8A8 comparator's HIP path (through the C ABI) with the CPU oracle.

Weight quantisation is integer work and must match bit for bit (codes and the fp32 row
scales).  The product's integer sums are exact, so the GPU value differs from the oracle's
fp64 value only by the epilogue's fp32 roundings: |y - y_ref| <= 4 * 2^-24 * |y_ref| (bf16
output adds 2^-9).  Small shapes cover several tiles and ragged tails in full; the model's
MLP shapes are checked on sampled rows and tokens.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_codebook_gemm_amd as mod
    mod.lib()
    return mod


def say(*a):
    print(*a, flush=True)


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def sample(n, count, seed):
    if n <= count:
        return np.arange(n)
    r = S.u64(seed, 79, count) % np.uint64(n)
    return np.unique(np.concatenate([[0, n - 1], r.astype(np.int64)]))


@functools.lru_cache(maxsize=None)
def oracle_w8(N, K, seed=0):
    W = S.weights(N, K, seed=seed)
    if N > 3:
        W[N // 2] = 0.0                  # a zero row: s_w = 0, codes 0
    return W, O.quantize_w8(W)


@functools.lru_cache(maxsize=None)
def oracle_acts(M, K, seed=0):
    x = S.activations(M, K, seed=seed, n_outliers=2)
    if M > 2:
        x[1] = 0.0                       # a zero token: s_x = 0
    return O.prepare(x)


def assert_close(y, yr, extra_rel=0.0):
    err = np.abs(y - yr)
    bound = (4 * U32 + extra_rel) * np.abs(yr)
    assert np.all(y[yr == 0] == 0)
    nz = yr != 0
    if nz.any():
        say(f"  max |y - y_ref| / |y_ref| = {(err[nz] / np.abs(yr[nz])).max():.3e}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("N,K,dt", [(256, 512, "f32"), (300, 768, "bf16"), (1, 256, "f32"), (37, 20736, "f32")])
def test_w8_quantize_bit_exact(w, N, K, dt):
    say(f"w8 quantize N={N} K={K} {dt}")
    W = S.weights(N, K, seed=N + K)
    if N > 3:
        W[2] = 0.0
    if dt == "bf16":
        bits = S.to_bf16_bits(W)
        win = gpu(bits.view(np.int16)).view(torch.bfloat16)
        W = S.bf16_bits_to_f32(bits)
    else:
        win = gpu(W)
    wq_ref, sw_ref = O.quantize_w8(W)
    L = w.w8a8_quantize_weight(win)
    torch.cuda.synchronize()
    assert np.array_equal(L.s_w.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))
    assert np.array_equal(L.w_q.cpu().numpy(), wq_ref)


def test_w8_quantize_full_size(w):
    N, K = S.MLP_GATE_UP
    say(f"w8 quantize full N={N} K={K}")
    W, (wq_ref, sw_ref) = oracle_w8(N, K, 5)
    L = w.w8a8_quantize_weight(gpu(W))
    torch.cuda.synchronize()
    assert np.array_equal(L.s_w.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))
    assert np.array_equal(L.w_q.cpu().numpy(), wq_ref)


def run(w, algo, N, K, M, rows=None, toks=None, out_dtype=torch.float32, seed=0):
    _, (wq, sw) = oracle_w8(N, K, seed)
    xq, sx = oracle_acts(M, K, seed)
    y = w.w8a8_linear(gpu(xq), gpu(sx), w.W8Linear(gpu(wq), gpu(sw)), out_dtype=out_dtype, algo=algo)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    rr = np.arange(N) if rows is None else rows
    tt = np.arange(M) if toks is None else toks
    y = y[np.ix_(tt, rr)]
    yr = O.linear_w8_ref(xq[tt], sx[tt], wq[rr], sw[rr])
    return y, yr


# M <= 4 with M*K <= 65536; ragged row counts, a row count below the CU count, and the
# longest rows the LDS staging holds
GEMV_CASES = [(256, 512, 1), (256, 512, 2), (256, 512, 3), (256, 512, 4), (1001, 768, 3), (1, 256, 1),
              (3000, 1280, 2), (8, 16384, 4), (64, 65536, 1)]


@pytest.mark.parametrize("N,K,M", GEMV_CASES)
def test_w8_gemv_parity(w, N, K, M):
    say(f"w8 gemv N={N} K={K} M={M}")
    assert_close(*run(w, w.ALGO_GEMV, N, K, M))


GEMM_CASES = [(256, 512, 4), (200, 768, 37), (300, 1024, 130), (128, 256, 128), (513, 1280, 257),
              (1, 256, 1), (1000, 2048, 5)]


@pytest.mark.parametrize("N,K,M", GEMM_CASES)
def test_w8_gemm_parity(w, N, K, M):
    say(f"w8 gemm N={N} K={K} M={M}")
    assert_close(*run(w, w.ALGO_MFMA_I8, N, K, M))


def test_w8_gemm_longest_rows_extreme_values(w):
    """K = 131072, the longest rows the format takes, with every product at +-127 x 127: the
    int32 sums reach 127^2 K = 2.11e9, just under 2^31, and must stay exact."""
    N, K, M = 200, 131072, 300
    say(f"w8 gemm extreme N={N} K={K} M={M}")
    wq = np.full((N, K), 127, dtype=np.int8)
    wq[1::2] = -127
    sw = np.full(N, 0.5, dtype=np.float32)
    xq = np.full((M, K), 127, dtype=np.int8)
    xq[::3] = -127
    sx = np.full(M, 0.25, dtype=np.float32)
    y = w.w8a8_linear(gpu(xq), gpu(sx), w.W8Linear(gpu(wq), gpu(sw)), algo=w.ALGO_MFMA_I8)
    torch.cuda.synchronize()
    rows, toks = sample(N, 24, 5), sample(M, 24, 6)
    y = y.cpu().numpy().astype(np.float64)[np.ix_(toks, rows)]
    yr = O.linear_w8_ref(xq[toks], sx[toks], wq[rows], sw[rows])
    assert np.abs(yr).max() == 127 * 127 * K * 0.5 * 0.25
    assert_close(y, yr)


@pytest.mark.parametrize("N,K,M,algo", [(17408, 5120, 1, 1), (5120, 17408, 2, 1), (17408, 5120, 2048, 2),
                                        (5120, 17408, 2048, 2)])
def test_w8_full_size_sampled(w, N, K, M, algo):
    say(f"w8 full N={N} K={K} M={M} algo={algo}")
    rows = sample(N, 96, N + 1)
    toks = sample(M, 48, M + 2)
    assert_close(*run(w, algo, N, K, M, rows=rows, toks=toks, seed=3))


@pytest.mark.parametrize("algo,M", [(1, 3), (2, 70)])
def test_w8_bf16_output(w, algo, M):
    say(f"w8 bf16 output algo={algo} M={M}")
    y, yr = run(w, algo, 300, 1024, M, out_dtype=torch.bfloat16)
    assert_close(y, yr, extra_rel=2.0 ** -8)


@pytest.mark.parametrize("algo,M", [(0, 1), (0, 4), (0, 5), (1, 2), (2, 33)])
def test_w8_deterministic(w, algo, M):
    say(f"w8 determinism algo={algo} M={M}")
    N, K = 777, 2560
    _, (wq, sw) = oracle_w8(N, K, 9)
    xq, sx = oracle_acts(M, K, 9)
    L = w.W8Linear(gpu(wq), gpu(sw))
    a = w.w8a8_linear(gpu(xq), gpu(sx), L, algo=algo)
    b = w.w8a8_linear(gpu(xq), gpu(sx), L, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert_close(a.cpu().numpy().astype(np.float64), O.linear_w8_ref(xq, sx, wq, sw))
