"""numpy front end of the CPU oracle (oracle/w4a8_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its Python binding.
Every function hands numpy arrays to the C oracle and returns numpy arrays; the
arithmetic and the citations of the model cards live in the C source.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = C.CDLL(_build.LIB)
        P = C.c_void_p
        i64, u64 = C.c_int64, C.c_uint64
        L.orc_num_threads.restype = C.c_int
        L.orc_fwht256.argtypes = [P]
        L.orc_rotate_rows.argtypes = [P, i64, i64, P]
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_decode.restype = C.c_double
        L.orc_e4m3_encode.argtypes = [C.c_float]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_splitmix64_at.argtypes = [u64, u64]
        L.orc_splitmix64_at.restype = u64
        L.orc_fit_sample.argtypes = [P, i64, u64, P]
        L.orc_fit_sample.restype = i64
        L.orc_lloyd_max16.argtypes = [P, i64, C.c_int, P, P]
        L.orc_lloyd_max16.restype = C.c_int
        L.orc_quantize_weight.argtypes = [P, i64, i64, u64, P, P, P, P, P]
        L.orc_quantize_weight.restype = C.c_int
        L.orc_prepare.argtypes = [P, i64, i64, P, P]
        L.orc_dequant.argtypes = [P, P, P, P, i64, i64, P]
        L.orc_linear_ref.argtypes = [P, P, i64, i64, P, P, P, P, i64, P, i64, P, i64, P, P]
        L.orc_codebook_i8.argtypes = [P, P, P]
        L.orc_linear_i8_ref.argtypes = [P, P, i64, i64, P, P, P, P, i64, P, i64, P, i64,
                                        P, P, P]
        L.orc_rq_table.argtypes = [P, P]
        L.orc_linear_rq_ref.argtypes = [P, P, i64, i64, P, P, P, P, i64, P, i64, P, i64, P]
        L.orc_quantize_w8.argtypes = [P, i64, i64, P, P]
        L.orc_linear_w8_ref.argtypes = [P, P, i64, i64, P, P, i64, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().orc_num_threads()


def fwht256(v) -> np.ndarray:
    """Rotate one 256-vector (fp32 fast transform, stages ascending, x 1/16)."""
    out = _c(v, np.float32).copy()
    assert out.shape == (256,)
    lib().orc_fwht256(_p(out))
    return out


def rotate_rows(W) -> np.ndarray:
    W = _c(W, np.float32)
    R, K = W.shape
    out = np.empty_like(W)
    lib().orc_rotate_rows(_p(W), R, K, _p(out))
    return out


def e4m3_decode(c: int) -> float:
    return lib().orc_e4m3_decode(int(c))


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(float(x))


def splitmix64_at(seed: int, i: int) -> int:
    return lib().orc_splitmix64_at(seed & (2**64 - 1), i)


def fit_sample(v, seed: int) -> np.ndarray:
    v = _c(v, np.float32).ravel()
    out = np.empty(min(v.size, 1 << 20), dtype=np.float32)
    S = lib().orc_fit_sample(_p(v), v.size, seed, _p(out))
    return out[:S]


def lloyd_max16(sample, max_iters: int = 100):
    """Returns (levels fp64 [16], number of updates, cell bounds int64 [17])."""
    s = _c(sample, np.float32).ravel()
    c = np.empty(16, dtype=np.float64)
    b = np.empty(17, dtype=np.int64)
    n = lib().orc_lloyd_max16(_p(s), s.size, int(max_iters), _p(c), _p(b))
    return c, n, b


def quantize_weight(W, seed: int = 0, want_v: bool = False):
    """Returns dict(packed int8 [N,K/2], s_rel uint8 [N,K/16], s_ch f32 [N], cb f32 [16],
    updates, and v f32 [N,K] if want_v)."""
    W = _c(W, np.float32)
    N, K = W.shape
    packed = np.empty((N, K // 2), dtype=np.int8)
    s_rel = np.empty((N, K // 16), dtype=np.uint8)
    s_ch = np.empty(N, dtype=np.float32)
    cb = np.empty(16, dtype=np.float32)
    v = np.empty((N, K), dtype=np.float32) if want_v else None
    n = lib().orc_quantize_weight(_p(W), N, K, seed & (2**64 - 1), _p(packed), _p(s_rel),
                                  _p(s_ch), _p(cb), _p(v))
    if n < 0:
        raise ValueError("K must be a positive multiple of 256")
    out = dict(packed=packed, s_rel=s_rel, s_ch=s_ch, cb=cb, updates=n)
    if want_v:
        out["v"] = v
    return out


def prepare(x):
    """fp32 activations [M,K] -> (x_q int8 [M,K], s_x f32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    xq = np.empty((M, K), dtype=np.int8)
    sx = np.empty(M, dtype=np.float32)
    lib().orc_prepare(_p(x), M, K, _p(xq), _p(sx))
    return xq, sx


def dequant(packed, s_rel, s_ch, cb) -> np.ndarray:
    packed = _c(packed, np.int8)
    N, K2 = packed.shape
    K = 2 * K2
    out = np.empty((N, K), dtype=np.float64)
    lib().orc_dequant(_p(packed), _p(_c(s_rel, np.uint8)), _p(_c(s_ch, np.float32)),
                      _p(_c(cb, np.float32)), N, K, _p(out))
    return out


def _subset(idx, n):
    if idx is None:
        return None, n
    idx = _c(idx, np.int64)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < n)
    return idx, idx.size


def linear_ref(xq, sx, packed, s_rel, s_ch, cb, rows=None, toks=None):
    """fp64 reference product.  Returns (y [ntok, nrow], A [ntok, nrow]) as float64."""
    xq = _c(xq, np.int8)
    M, K = xq.shape
    packed = _c(packed, np.int8)
    N = packed.shape[0]
    rows, nrow = _subset(rows, N)
    toks, ntok = _subset(toks, M)
    y = np.empty((ntok, nrow), dtype=np.float64)
    A = np.empty((ntok, nrow), dtype=np.float64)
    lib().orc_linear_ref(_p(xq), _p(_c(sx, np.float32)), M, K, _p(packed),
                         _p(_c(s_rel, np.uint8)), _p(_c(s_ch, np.float32)),
                         _p(_c(cb, np.float32)), N, _p(rows), nrow, _p(toks), ntok,
                         _p(y), _p(A))
    return y, A


def codebook_i8(cb):
    cb = _c(cb, np.float32)
    s = np.empty(1, dtype=np.float32)
    q = np.empty(16, dtype=np.int8)
    lib().orc_codebook_i8(_p(cb), _p(s), _p(q))
    return float(s[0]), q


def linear_i8_ref(xq, sx, packed, s_rel, s_ch, cb, rows=None, toks=None, want_p=False):
    """int8-codebook product.  Returns (y8, A8[, P int32 [ntok, nrow, K/16]])."""
    xq = _c(xq, np.int8)
    M, K = xq.shape
    packed = _c(packed, np.int8)
    N = packed.shape[0]
    rows, nrow = _subset(rows, N)
    toks, ntok = _subset(toks, M)
    y = np.empty((ntok, nrow), dtype=np.float64)
    A = np.empty((ntok, nrow), dtype=np.float64)
    P = np.empty((ntok, nrow, K // 16), dtype=np.int32) if want_p else None
    lib().orc_linear_i8_ref(_p(xq), _p(_c(sx, np.float32)), M, K, _p(packed),
                            _p(_c(s_rel, np.uint8)), _p(_c(s_ch, np.float32)),
                            _p(_c(cb, np.float32)), N, _p(rows), nrow, _p(toks), ntok,
                            _p(y), _p(A), _p(P))
    return (y, A, P) if want_p else (y, A)


def rq_table(cb) -> np.ndarray:
    """Requantised int8 weight table t [256 e4m3 codes, 16 levels]."""
    cb = _c(cb, np.float32)
    t = np.empty((256, 16), dtype=np.int8)
    lib().orc_rq_table(_p(cb), _p(t))
    return t


def linear_rq_ref(xq, sx, packed, s_rel, s_ch, cb, rows=None, toks=None):
    """Product on requantised int8 weights: y fp32 [ntok, nrow], exactly as defined."""
    xq = _c(xq, np.int8)
    M, K = xq.shape
    packed = _c(packed, np.int8)
    N = packed.shape[0]
    rows, nrow = _subset(rows, N)
    toks, ntok = _subset(toks, M)
    y = np.empty((ntok, nrow), dtype=np.float32)
    lib().orc_linear_rq_ref(_p(xq), _p(_c(sx, np.float32)), M, K, _p(packed),
                            _p(_c(s_rel, np.uint8)), _p(_c(s_ch, np.float32)),
                            _p(_c(cb, np.float32)), N, _p(rows), nrow, _p(toks), ntok, _p(y))
    return y


def quantize_w8(W):
    """W8A8 comparator weights: rotated rows, per-row int8.  Returns (w_q int8 [N, K], s_w fp32 [N])."""
    W = _c(W, np.float32)
    N, K = W.shape
    assert K % 256 == 0
    wq = np.empty((N, K), dtype=np.int8)
    sw = np.empty((N,), dtype=np.float32)
    lib().orc_quantize_w8(_p(W), N, K, _p(wq), _p(sw))
    return wq, sw


def linear_w8_ref(xq, sx, wq, sw):
    """W8A8 comparator product in fp64 (exact integer dot products): y [M, N]."""
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    lib().orc_linear_w8_ref(_p(xq), _p(_c(sx, np.float32)), M, K, _p(wq), _p(_c(sw, np.float32)), N, _p(y))
    return y
