"""Several layers per call (w4a8_linear_multi, w4a8_forward_multi) on the GPU.

Each layer's output must be bit-identical to the single-layer call it stands for (the
per-row arithmetic does not depend on how the rows are shared between workgroups), and the
prepared activations bit-exact with the oracle.  One case is also gated against the oracle
directly.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# row counts of the layers of one call: ragged, small and large, below and above one row
# per CU
NS = [5120, 1000, 17, 2048, 300, 4096, 64, 777]


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


@functools.lru_cache(maxsize=None)
def oracle_layer(N, K, seed):
    return O.quantize_weight(S.weights(N, K, seed=seed), seed=seed)


def layers_for(w, G, K):
    qs = [oracle_layer(NS[g], K, 20 + g) for g in range(G)]
    return qs, [w.QuantizedLinear(gpu(q["packed"]), gpu(q["s_rel"]), gpu(q["s_ch"]), gpu(q["cb"])) for q in qs]


@pytest.mark.parametrize("M,K,G", [(1, 5120, 1), (1, 5120, 4), (2, 2560, 8), (3, 1024, 3), (4, 10240, 2),
                                   (1, 256, 8), (8, 768, 3)])
def test_linear_multi_matches_single(w, M, K, G):
    say(f"linear_multi M={M} K={K} G={G}")
    qs, Ls = layers_for(w, G, K)
    x = S.activations(M, K, seed=M + K, n_outliers=2)
    xq, sx = O.prepare(x)
    xg, sg = gpu(xq), gpu(sx)
    ys = w.linear_multi(xg, sg, Ls)
    ref = [w.linear(xg, sg, L) for L in Ls]
    torch.cuda.synchronize()
    for g in range(G):
        assert torch.equal(ys[g], ref[g]), g
    # the first layer against the oracle as well
    q = qs[0]
    yr, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    err = np.abs(ys[0].cpu().numpy().astype(np.float64) - yr)
    assert np.all(err <= 4e-3 * A)


@pytest.mark.parametrize("M,K,G,N,dt", [(8, 5120, 4, 5120, "f32"), (40, 1024, 3, 1000, "bf16"), (4, 2048, 2, 77, "f32"),
                                        (64, 512, 8, 300, "f32"), (17, 8192, 2, 5120, "bf16")])
def test_linear_multi_same_rows_one_launch(w, M, K, G, N, dt):
    # layers with one row count run as one batched-decode launch; each output must match
    # the single-layer call bit for bit
    say(f"linear_multi same N={N} M={M} K={K} G={G} {dt}")
    qs = [oracle_layer(N, K, 40 + g) for g in range(G)]
    Ls = [w.QuantizedLinear(gpu(q["packed"]), gpu(q["s_rel"]), gpu(q["s_ch"]), gpu(q["cb"])) for q in qs]
    x = S.activations(M, K, seed=7 * M + K, n_outliers=2)
    xq, sx = O.prepare(x)
    xg, sg = gpu(xq), gpu(sx)
    odt = torch.bfloat16 if dt == "bf16" else torch.float32
    assert w.linear_pick(M, N, K) == w.ALGO_MFMA_SKINNY
    ys = w.linear_multi(xg, sg, Ls, out_dtype=odt)
    ref = [w.linear(xg, sg, L, out_dtype=odt) for L in Ls]
    torch.cuda.synchronize()
    for g in range(G):
        assert torch.equal(ys[g], ref[g]), g
    # the last layer against the oracle as well
    q = qs[-1]
    yr, A = O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
    err = np.abs(ys[-1].float().cpu().numpy().astype(np.float64) - yr)
    bound = 4e-3 * A + (np.abs(yr) * 2.0 ** -8 if dt == "bf16" else 0.0)
    assert np.all(err <= bound)


@pytest.mark.parametrize("M,K,G,dt", [(1, 5120, 4, "f32"), (1, 17408, 2, "bf16"), (2, 5120, 3, "f32"),
                                      (2, 1024, 8, "bf16"), (1, 33024, 2, "f32"), (3, 512, 2, "f32")])
def test_forward_multi_matches_single(w, M, K, G, dt):
    say(f"forward_multi M={M} K={K} G={G} {dt}")
    qs, Ls = layers_for(w, G, K)
    x = S.activations(M, K, seed=3 * M + K, n_outliers=2)
    if dt == "bf16":
        bits = S.to_bf16_bits(x)
        xin = gpu(bits.view(np.int16)).view(torch.bfloat16)
        x = S.bf16_bits_to_f32(bits)
    else:
        xin = gpu(x)
    xq_ref, sx_ref = O.prepare(x)
    x_q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s_x = torch.empty((M,), dtype=torch.float32, device=DEV)
    ys = w.forward_multi(xin, Ls, x_q=x_q, s_x=s_x)
    ref = [w.forward(xin, L) for L in Ls]
    torch.cuda.synchronize()
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(x_q.cpu().numpy(), xq_ref)
    for g in range(G):
        assert torch.equal(ys[g], ref[g]), g


def test_multi_bf16_outputs_and_rejects(w):
    say("multi bf16 outputs and argument errors")
    qs, Ls = layers_for(w, 3, 1024)
    x = gpu(S.activations(1, 1024, seed=5))
    ys = w.forward_multi(x, Ls, out_dtype=torch.bfloat16)
    ref = [w.forward(x, L, out_dtype=torch.bfloat16) for L in Ls]
    torch.cuda.synchronize()
    for a, b in zip(ys, ref):
        assert torch.equal(a, b)
    with pytest.raises(ValueError):
        w.forward_multi(x, Ls * 3)           # 9 layers
    with pytest.raises(ValueError):          # outputs of mixed dtypes
        w.forward_multi(x, Ls[:2], outs=[torch.empty((1, NS[0]), device=DEV),
                                         torch.empty((1, NS[1]), dtype=torch.bfloat16, device=DEV)])
