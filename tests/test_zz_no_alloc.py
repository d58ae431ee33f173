"""The no-allocation quantiser entry point (w4a8_quantize_weight_noalloc) against the one
with a caller workspace (w4a8_quantize_weight), through the C ABI on the GPU.

Both run the same kernels, so all four outputs must be identical bit for bit.  Calls come in
a row on one device, each smaller than the one before (the static scratch keeps the last
call's contents, which the next call must not depend on): a full MLP matrix (sampled fit),
a smaller sampled one from bf16, then one small enough that the fit takes every value.  The
last call is also checked against the CPU oracle.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_codebook_gemm_amd as mod
    mod.lib()
    return mod


def outputs(n, k):
    return (torch.empty((n, k // 2), dtype=torch.int8, device=DEV), torch.empty((n, k // 16), dtype=torch.uint8, device=DEV),
            torch.empty((n,), dtype=torch.float32, device=DEV), torch.empty((16,), dtype=torch.float32, device=DEV))


def run_pair(w, W, seed):
    n, k = W.shape
    dt = w.BF16 if W.dtype == torch.bfloat16 else w.F32
    stream = torch.cuda.current_stream().cuda_stream
    a = outputs(n, k)
    ws = torch.empty((w.quantize_weight_workspace(n, k),), dtype=torch.uint8, device=DEV)
    st = w.lib().w4a8_quantize_weight(W.data_ptr(), dt, n, k, seed, *(t.data_ptr() for t in a), ws.data_ptr(),
                                      ws.numel(), stream)
    assert st == 0, st
    b = outputs(n, k)
    for t in b:
        t.fill_(0x55 if t.dtype in (torch.int8, torch.uint8) else 7.0)
    st = w.lib().w4a8_quantize_weight_noalloc(W.data_ptr(), dt, n, k, seed, *(t.data_ptr() for t in b), stream)
    assert st == 0, st
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.int8 else x,
                           y.view(torch.uint8) if y.dtype == torch.int8 else y)
    return b


def test_noalloc_matches_workspace_entry_point(w):
    shapes = [(S.MLP_GATE_UP, torch.float32, 0), ((2048, 1024), torch.bfloat16, 42), ((300, 768), torch.float32, 7)]
    last = None
    for (n, k), dtype, seed in shapes:
        print(f"noalloc quantize N={n} K={k} {dtype} seed={seed}", flush=True)
        W = S.weights(n, k, seed=seed)
        Wg = torch.from_numpy(W).to(DEV)
        if dtype == torch.bfloat16:
            Wg = torch.from_numpy(S.to_bf16_bits(W).view(np.int16)).to(DEV).view(torch.bfloat16)
            W = S.bf16_bits_to_f32(S.to_bf16_bits(W))
        last = (W, seed, run_pair(w, Wg, seed))
    W, seed, (packed, s_rel, s_ch, cb) = last
    q = O.quantize_weight(W, seed=seed)
    assert np.array_equal(packed.cpu().numpy(), q["packed"])
    assert np.array_equal(s_rel.cpu().numpy(), q["s_rel"])
    assert np.array_equal(s_ch.cpu().numpy().view(np.uint32), q["s_ch"].view(np.uint32))
    assert np.array_equal(cb.cpu().numpy().view(np.uint32), q["cb"].view(np.uint32))


def test_noalloc_argument_errors(w):
    """Validation happens before any launch: a NULL output, a K that is not a multiple of 256,
    an unknown dtype."""
    W = torch.zeros((4, 256), device=DEV)
    o = outputs(4, 256)
    f = w.lib().w4a8_quantize_weight_noalloc
    s = torch.cuda.current_stream().cuda_stream
    assert f(W.data_ptr(), w.F32, 4, 256, 0, None, *(t.data_ptr() for t in o[1:]), s) == 1
    assert f(W.data_ptr(), w.F32, 4, 200, 0, *(t.data_ptr() for t in o), s) == 2
    assert f(W.data_ptr(), 9, 4, 256, 0, *(t.data_ptr() for t in o), s) == 3
