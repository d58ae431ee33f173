"""The C ABI without a GPU: the library loads, exports every symbol include/w4a8.h
declares, and every argument-validation error is returned before any HIP call."""
import ctypes as C
import os
import re

import pytest
import torch  # noqa: F401  (binds the library's HIP runtime to torch's)

import w4a8_codebook_gemm_amd as w
from conftest import ROOT

FAKE = 0x10000  # a 16-byte aligned non-null address that is never dereferenced
MIS = FAKE + 8  # misaligned


def header_functions():
    text = open(os.path.join(ROOT, "include", "w4a8.h")).read()
    return re.findall(r"W4A8_API\s+[\w\s\*]+?\b(w4a8_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w.LIB_PATH):
        pytest.skip("library not built")
    return w.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 16 and set(names) == set(w.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_exports_nothing_else():
    out = os.popen(f"nm -D --defined-only {w.LIB_PATH}").read()
    text = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert sorted(text) == sorted(w.EXPORTS)


def test_version_and_status_strings(L):
    assert L.w4a8_version() == 100
    for s in range(8):
        assert len(L.w4a8_status_string(s)) > 0
    assert L.w4a8_status_string(99) == b"unknown status"


def test_workspace_size_and_pick(L):
    # the fit sample's uint32 keys (padded to a power of two, at least 2048) and its fp64
    # prefix sums, each rounded up to 256 bytes: no term grows with N * K past 2^20
    up = lambda b: (b + 255) // 256 * 256
    assert L.w4a8_quantize_weight_workspace(256, 512) == up(131072 * 4) + up((131072 + 1) * 8)
    assert L.w4a8_quantize_weight_workspace(1, 256) == up(2048 * 4) + up(257 * 8)
    assert L.w4a8_quantize_weight_workspace(300, 768) == up(262144 * 4) + up((300 * 768 + 1) * 8)
    full = up((1 << 20) * 4) + up(((1 << 20) + 1) * 8)
    assert full == 12583168
    assert L.w4a8_quantize_weight_workspace(17408, 5120) == full
    assert L.w4a8_quantize_weight_workspace(1 << 20, 1 << 16) == full
    for bad in [(0, 512), (4, 4304), (4, 100), (-1, 256), (4, 0)]:
        assert L.w4a8_quantize_weight_workspace(*bad) == 0
    assert L.w4a8_linear_pick(1, 17408, 5120) == w.ALGO_GEMV
    assert L.w4a8_linear_pick(2, 5120, 17408) == w.ALGO_GEMV
    assert L.w4a8_linear_pick(4, 17408, 5120) == w.ALGO_MFMA_SKINNY
    assert L.w4a8_linear_pick(4, 5120, 5120) == w.ALGO_MFMA_SKINNY
    assert L.w4a8_linear_pick(3, 17408, 5120) == w.ALGO_GEMV
    assert L.w4a8_linear_pick(3, 5120, 17408) == w.ALGO_MFMA_SKINNY
    assert L.w4a8_linear_pick(5, 17408, 5120) == w.ALGO_MFMA_SKINNY
    assert L.w4a8_linear_pick(64, 5120, 17408) == w.ALGO_MFMA_SKINNY
    assert L.w4a8_linear_pick(65, 5120, 17408) == w.ALGO_MFMA_F16
    assert L.w4a8_linear_pick(2048, 17408, 5120) == w.ALGO_MFMA_F16
    assert L.w4a8_linear_pick(1, 1, 4304) == -2


def lin(L, M=4, K=512, N=256, ptrs=None, ydt=0, algo=0):
    p = dict(xq=FAKE, sx=FAKE, pk=FAKE, sr=FAKE, sc=FAKE, cb=FAKE, y=FAKE)
    p.update(ptrs or {})
    return L.w4a8_linear_algo(p["xq"], p["sx"], M, K, p["pk"], p["sr"], p["sc"], p["cb"], N, p["y"], ydt,
                              algo, None)


def test_linear_validation(L):
    for k in ("xq", "sx", "pk", "sr", "sc", "cb", "y"):
        assert lin(L, ptrs={k: 0}) == 1
    for M, K, N in [(0, 512, 4), (4, 4304, 4), (4, 128, 4), (4, 512, 0), (-3, 512, 4), (4, 0, 4)]:
        assert lin(L, M=M, K=K, N=N) == 2
    assert lin(L, ydt=7) == 3
    assert lin(L, algo=9) == 3
    for k in ("xq", "sx", "pk", "sr", "sc", "cb", "y"):
        assert lin(L, ptrs={k: MIS}) == 4
    assert lin(L, M=8, K=5120, algo=w.ALGO_GEMV) == 2  # outside the GEMV's range
    assert lin(L, M=65, K=512, algo=w.ALGO_MFMA_SKINNY) == 2  # outside the skinny kernel's
    assert lin(L, algo=7) == 3
    assert lin(L, M=4, K=131328, algo=w.ALGO_MFMA_RQ) == 2  # the int32 sum would not be exact
    huge = (1 << 31) - 1                                     # 2^31 - 1 tokens and rows: too many tiles
    for a in (w.ALGO_MFMA_I8, w.ALGO_MFMA_F16, w.ALGO_MFMA_RQ, w.ALGO_MFMA_I8_FOLD):
        assert lin(L, M=huge, N=huge, algo=a) == 2
    assert L.w4a8_linear(0, FAKE, 4, 512, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, None) == 1


def test_linear_ws_validation(L):
    """The workspace entry points validate like w4a8_linear, plus the workspace's alignment,
    before any HIP call; a shape the batched-decode kernel does not take needs no workspace."""
    ws = lambda wsp=FAKE, nb=1 << 20, **kw: L.w4a8_linear_ws(
        FAKE if "xq" not in kw else kw["xq"], FAKE, kw.get("M", 4), kw.get("K", 512), FAKE, FAKE, FAKE, FAKE,
        kw.get("N", 4), FAKE, kw.get("ydt", 0), wsp, nb, None)
    assert ws(xq=0) == 1
    for M, K, N in [(0, 512, 4), (4, 4304, 4), (4, 128, 4), (4, 512, 0)]:
        assert ws(M=M, K=K, N=N) == 2
    assert ws(ydt=7) == 3
    assert ws(wsp=MIS) == 4
    for M, K, N in [(0, 512, 4), (4, 100, 4), (4, 512, 0)]:
        assert L.w4a8_linear_workspace_bytes(M, N, K) == -2
    assert L.w4a8_linear_workspace_bytes(1, 5120, 5120) == 0     # the GEMV
    assert L.w4a8_linear_workspace_bytes(2048, 5120, 5120) == 0  # a prefill GEMM


def test_prepare_and_quantize_validation(L):
    assert L.w4a8_prepare_activation(0, 0, 4, 512, FAKE, FAKE, None) == 1
    assert L.w4a8_prepare_activation(FAKE, 0, 4, 300, FAKE, FAKE, None) == 2
    assert L.w4a8_prepare_activation(FAKE, 5, 4, 512, FAKE, FAKE, None) == 3
    assert L.w4a8_prepare_activation(MIS, 0, 4, 512, FAKE, FAKE, None) == 4
    need = L.w4a8_quantize_weight_workspace(8, 256)
    q = L.w4a8_quantize_weight
    assert q(0, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 1
    assert q(FAKE, 0, 8, 4304, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 2
    assert q(FAKE, 2, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 3
    assert q(FAKE, 0, 8, 256, 0, MIS, FAKE, FAKE, FAKE, FAKE, need, None) == 4
    assert q(FAKE, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 5
    assert q(FAKE, 0, 8, 256, 0, FAKE, FAKE, FAKE, FAKE, 0, need, None) == 5


def test_binding_refuses_cpu_tensors_and_bad_shapes():
    x = torch.zeros(4, 512)
    with pytest.raises(ValueError):
        w.prepare_activation(x)
    with pytest.raises(ValueError):
        w.quantize_weight(torch.zeros(4, 512, 3))


def test_binding_raises_loudly_without_library(monkeypatch):
    monkeypatch.setattr(w, "_lib", None)
    monkeypatch.setattr(w, "LIB_PATH", "/nonexistent/libw4a8.so")
    with pytest.raises(RuntimeError):
        w.lib()


def test_forward_validation(L):
    f = L.w4a8_forward
    args = lambda **kw: [kw.get("x", FAKE), kw.get("xdt", 0), kw.get("M", 1), kw.get("K", 512), FAKE, FAKE, FAKE,
                         FAKE, kw.get("N", 256), FAKE, 0, kw.get("xq", FAKE), kw.get("sx", FAKE), None]
    assert f(*args(x=0)) == 1
    assert f(*args(xq=0)) == 1
    assert f(*args(sx=0)) == 1
    assert f(*args(K=4304)) == 2
    assert f(*args(M=0)) == 2
    assert f(*args(xdt=4)) == 3
    assert f(*args(x=MIS)) == 4
    assert f(*args(xq=MIS)) == 4


def test_w8a8_validation(L):
    q = L.w4a8_w8a8_quantize_weight
    assert q(0, 0, 8, 256, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 8, 4304, FAKE, FAKE, None) == 2
    assert q(FAKE, 0, 8, 131072 + 256, FAKE, FAKE, None) == 2   # exact int32 sums need K <= 2^17
    assert q(FAKE, 0, 0, 256, FAKE, FAKE, None) == 2
    assert q(FAKE, 2, 8, 256, FAKE, FAKE, None) == 3
    assert q(FAKE, 0, 8, 256, MIS, FAKE, None) == 4

    def lin8(M=4, K=512, N=256, ydt=0, algo=0, **ptrs):
        p = dict(xq=FAKE, sx=FAKE, wq=FAKE, sw=FAKE, y=FAKE)
        p.update(ptrs)
        return L.w4a8_w8a8_linear(p["xq"], p["sx"], M, K, p["wq"], p["sw"], N, p["y"], ydt, algo, None)

    for k in ("xq", "sx", "wq", "sw", "y"):
        assert lin8(**{k: 0}) == 1
        assert lin8(**{k: MIS}) == 4
    for M, K, N in [(0, 512, 4), (4, 300, 4), (4, 512, 0), (4, 131072 + 256, 4)]:
        assert lin8(M=M, K=K, N=N) == 2
    assert lin8(ydt=2) == 3
    assert lin8(algo=w.ALGO_MFMA_F16) == 3
    assert lin8(algo=w.ALGO_MFMA_SKINNY) == 3
    assert lin8(M=5, algo=w.ALGO_GEMV) == 2              # GEMV: M <= 4
    assert lin8(M=4, K=16640, algo=w.ALGO_GEMV) == 2     # GEMV: M*K <= 65536


def test_multi_validation(L):
    def table(G, **bad):
        t = (w.Layer * max(G, 1))()
        for g in range(max(G, 1)):
            t[g] = w.Layer(FAKE, FAKE, FAKE, FAKE, 256, FAKE)
        for k, v in bad.items():
            setattr(t[0], k, v)
        return t

    def lin(G=2, t=None, M=1, K=512, ydt=0, xq=FAKE):
        t = table(G) if t is None else t
        return L.w4a8_linear_multi(xq, FAKE, M, K, G, C.addressof(t), ydt, None)

    assert L.w4a8_linear_multi(FAKE, FAKE, 1, 512, 2, None, 0, None) == 1
    assert lin(G=0) == 2 and lin(G=9) == 2
    assert lin(t=table(2, packed=0)) == 1
    assert lin(t=table(2, y=MIS)) == 4
    assert lin(t=table(2, N=0)) == 2
    assert lin(K=300) == 2
    assert lin(ydt=5) == 3
    assert lin(xq=0) == 1
    f = L.w4a8_forward_multi
    t = table(2)
    assert f(0, 0, 1, 512, 2, C.addressof(t), 0, FAKE, FAKE, None) == 1
    assert f(FAKE, 4, 1, 512, 2, C.addressof(t), 0, FAKE, FAKE, None) == 3
    assert f(MIS, 0, 1, 512, 2, C.addressof(t), 0, FAKE, FAKE, None) == 4
    assert f(FAKE, 0, 1, 512, 2, C.addressof(t), 0, 0, FAKE, None) == 1
