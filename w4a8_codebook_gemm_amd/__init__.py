"""Python binding of libw4a8.so, the MI355X (gfx950) W4A8 codebook linear layer.

Argument marshalling only: every function checks tensor placement, dtype and layout, then
passes raw device pointers, sizes and the current HIP stream to the C ABI declared in
include/w4a8.h.  All arithmetic runs in the library's HIP kernels; PyTorch provides device
memory and streams.  There is no fallback: if the library is missing or fails to load,
every call raises.

The layer format (model cards "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", section
"Format"; "Qwen3.8-27B-W4A8 (for ComfyUI)", section "Model Overview"):
  packed int8 [N, K/2], s_rel uint8 [N, K/16] (E4M3FN bits), s_channel fp32 [N],
  codebook fp32 [16].
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a8.so")

F32, BF16 = 0, 1
ALGO_AUTO, ALGO_GEMV, ALGO_MFMA_I8, ALGO_MFMA_F16, ALGO_MFMA_SKINNY, ALGO_MFMA_RQ = 0, 1, 2, 3, 4, 5
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_ALIGN",
          5: "ERR_WORKSPACE", 6: "ERR_HIP", 7: "ERR_DEVICE"}
EXPORTS = ("w4a8_version", "w4a8_status_string", "w4a8_quantize_weight_workspace",
           "w4a8_quantize_weight", "w4a8_prepare_activation", "w4a8_linear",
           "w4a8_linear_algo", "w4a8_linear_pick", "w4a8_forward", "w4a8_linear_multi",
           "w4a8_forward_multi", "w4a8_w8a8_quantize_weight", "w4a8_w8a8_linear")
MAX_GROUP = 8


class Layer(C.Structure):
    """w4a8_layer: one layer's device pointers, rows and output pointer."""
    _fields_ = [("packed", C.c_void_p), ("s_rel", C.c_void_p), ("s_channel", C.c_void_p),
                ("codebook", C.c_void_p), ("N", C.c_int64), ("y", C.c_void_p)]


class W4A8Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({lib().w4a8_status_string(status).decode()})")


_lib = None


def lib():
    """The loaded C library (torch is imported first so HIP resolves to torch's runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python w4a8_codebook_gemm_amd/build.py")
        L = C.CDLL(LIB_PATH)
        P, i64, u64, i32, sz = C.c_void_p, C.c_int64, C.c_uint64, C.c_int, C.c_size_t
        L.w4a8_version.restype = i32
        L.w4a8_status_string.argtypes = [i32]
        L.w4a8_status_string.restype = C.c_char_p
        L.w4a8_quantize_weight_workspace.argtypes = [i64, i64]
        L.w4a8_quantize_weight_workspace.restype = sz
        L.w4a8_quantize_weight.argtypes = [P, i32, i64, i64, u64, P, P, P, P, P, sz, P]
        L.w4a8_quantize_weight.restype = i32
        L.w4a8_prepare_activation.argtypes = [P, i32, i64, i64, P, P, P]
        L.w4a8_prepare_activation.restype = i32
        L.w4a8_linear.argtypes = [P, P, i64, i64, P, P, P, P, i64, P, i32, P]
        L.w4a8_linear.restype = i32
        L.w4a8_linear_algo.argtypes = [P, P, i64, i64, P, P, P, P, i64, P, i32, i32, P]
        L.w4a8_linear_algo.restype = i32
        L.w4a8_linear_pick.argtypes = [i64, i64, i64]
        L.w4a8_linear_pick.restype = i32
        L.w4a8_forward.argtypes = [P, i32, i64, i64, P, P, P, P, i64, P, i32, P, P, P]
        L.w4a8_forward.restype = i32
        L.w4a8_linear_multi.argtypes = [P, P, i64, i64, i32, P, i32, P]
        L.w4a8_linear_multi.restype = i32
        L.w4a8_forward_multi.argtypes = [P, i32, i64, i64, i32, P, i32, P, P, P]
        L.w4a8_forward_multi.restype = i32
        L.w4a8_w8a8_quantize_weight.argtypes = [P, i32, i64, i64, P, P, P]
        L.w4a8_w8a8_quantize_weight.restype = i32
        L.w4a8_w8a8_linear.argtypes = [P, P, i64, i64, P, P, i64, P, i32, i32, P]
        L.w4a8_w8a8_linear.restype = i32
        _lib = L
    return _lib


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _fdtype(t: torch.Tensor) -> int:
    return BF16 if t.dtype == torch.bfloat16 else F32


def _check(status: int, what: str):
    if status != 0:
        raise W4A8Error(status, what)


@dataclass
class QuantizedLinear:
    """One quantised layer: the four tensors of the format (N rows, K input features)."""
    packed: torch.Tensor      # int8 [N, K/2]
    s_rel: torch.Tensor       # uint8 [N, K/16], E4M3FN bit patterns
    s_channel: torch.Tensor   # float32 [N]
    codebook: torch.Tensor    # float32 [16]

    @property
    def out_features(self) -> int:
        return self.packed.shape[0]

    @property
    def in_features(self) -> int:
        return self.packed.shape[1] * 2

    def __call__(self, x: torch.Tensor, out_dtype=torch.float32, algo: int = ALGO_AUTO):
        if algo == ALGO_AUTO:
            return forward(x, self, out_dtype=out_dtype)
        x_q, s_x = prepare_activation(x)
        return linear(x_q, s_x, self, out_dtype=out_dtype, algo=algo)


def quantize_weight_workspace(n: int, k: int) -> int:
    return int(lib().w4a8_quantize_weight_workspace(n, k))


def quantize_weight(w: torch.Tensor, seed: int = 0, workspace: torch.Tensor | None = None) -> QuantizedLinear:
    """Quantise a [N, K] fp32/bf16 weight on the GPU (asynchronous on the current stream)."""
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    wp = _dev(w, "w", (torch.float32, torch.bfloat16))
    dev = w.device
    packed = torch.empty((n, k // 2), dtype=torch.int8, device=dev)
    s_rel = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    s_ch = torch.empty((n,), dtype=torch.float32, device=dev)
    cb = torch.empty((16,), dtype=torch.float32, device=dev)
    need = quantize_weight_workspace(n, k)
    if need == 0:
        _check(2, "w4a8_quantize_weight")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    _check(lib().w4a8_quantize_weight(wp, _fdtype(w), n, k, seed & (2**64 - 1), packed.data_ptr(),
                                      s_rel.data_ptr(), s_ch.data_ptr(), cb.data_ptr(),
                                      _dev(workspace, "workspace", (torch.uint8,)),
                                      workspace.numel(), _stream()), "w4a8_quantize_weight")
    return QuantizedLinear(packed, s_rel, s_ch, cb)


def prepare_activation(x: torch.Tensor, out=None):
    """Rotate and quantise activations [M, K] fp32/bf16 -> (x_q int8 [M, K], s_x fp32 [M])."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    xp = _dev(x, "x", (torch.float32, torch.bfloat16))
    if out is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
        s_x = torch.empty((m,), dtype=torch.float32, device=x.device)
    else:
        x_q, s_x = out
    _check(lib().w4a8_prepare_activation(xp, _fdtype(x), m, k, _dev(x_q, "x_q", (torch.int8,)),
                                         _dev(s_x, "s_x", (torch.float32,)), _stream()),
           "w4a8_prepare_activation")
    return x_q, s_x


def linear(x_q: torch.Tensor, s_x: torch.Tensor, layer: QuantizedLinear, out_dtype=torch.float32,
           algo: int = ALGO_AUTO, out: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] = the quantised product of prepared activations with one layer.

    algo: ALGO_AUTO (what w4a8_linear picks), ALGO_GEMV, ALGO_MFMA_SKINNY, ALGO_MFMA_F16,
    ALGO_MFMA_I8 (exact per-16 fold) or ALGO_MFMA_RQ (weights requantised to int8: an
    approximation of the product, see w4a8.h)."""
    m, k = x_q.shape
    n = layer.packed.shape[0]
    if (tuple(layer.packed.shape) != (n, k // 2) or tuple(layer.s_rel.shape) != (n, k // 16)
            or tuple(layer.s_channel.shape) != (n,) or tuple(layer.codebook.shape) != (16,)
            or tuple(s_x.shape) != (m,)):
        raise ValueError(f"inconsistent shapes: x_q {tuple(x_q.shape)}, s_x {tuple(s_x.shape)}, "
                         f"packed {tuple(layer.packed.shape)}, s_rel {tuple(layer.s_rel.shape)}, "
                         f"s_channel {tuple(layer.s_channel.shape)}, codebook {tuple(layer.codebook.shape)}")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x_q.device)
    yp = _dev(out, "y", (torch.float32, torch.bfloat16))
    _check(lib().w4a8_linear_algo(
        _dev(x_q, "x_q", (torch.int8,)), _dev(s_x, "s_x", (torch.float32,)), m, k,
        _dev(layer.packed, "packed", (torch.int8,)), _dev(layer.s_rel, "s_rel", (torch.uint8,)),
        _dev(layer.s_channel, "s_channel", (torch.float32,)),
        _dev(layer.codebook, "codebook", (torch.float32,)), n, yp, _fdtype(out), algo, _stream()),
        "w4a8_linear")
    return out


def forward(x: torch.Tensor, layer: QuantizedLinear, out_dtype=torch.float32, out=None,
            x_q: torch.Tensor | None = None, s_x: torch.Tensor | None = None) -> torch.Tensor:
    """prepare_activation + linear in one call (one kernel launch for decode sizes).
    x_q [M, K] int8 and s_x [M] fp32 receive the prepared activations."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    n = layer.packed.shape[0]
    if (tuple(layer.packed.shape) != (n, k // 2) or tuple(layer.s_rel.shape) != (n, k // 16)
            or tuple(layer.s_channel.shape) != (n,) or tuple(layer.codebook.shape) != (16,)):
        raise ValueError("layer tensors do not match x's in_features")
    xp = _dev(x, "x", (torch.float32, torch.bfloat16))
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty((m,), dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check(lib().w4a8_forward(xp, _fdtype(x), m, k, _dev(layer.packed, "packed", (torch.int8,)),
                              _dev(layer.s_rel, "s_rel", (torch.uint8,)),
                              _dev(layer.s_channel, "s_channel", (torch.float32,)),
                              _dev(layer.codebook, "codebook", (torch.float32,)), n,
                              _dev(out, "y", (torch.float32, torch.bfloat16)), _fdtype(out),
                              _dev(x_q, "x_q", (torch.int8,)), _dev(s_x, "s_x", (torch.float32,)),
                              _stream()), "w4a8_forward")
    return out


def _layer_table(layers, m, k, out_dtype, outs):
    if not 1 <= len(layers) <= MAX_GROUP:
        raise ValueError(f"1 to {MAX_GROUP} layers per call, got {len(layers)}")
    if outs is None:
        outs = [None] * len(layers)
    table = (Layer * len(layers))()
    ys = []
    for g, (L, y) in enumerate(zip(layers, outs)):
        n = L.packed.shape[0]
        if (tuple(L.packed.shape) != (n, k // 2) or tuple(L.s_rel.shape) != (n, k // 16)
                or tuple(L.s_channel.shape) != (n,) or tuple(L.codebook.shape) != (16,)):
            raise ValueError(f"layer {g}: tensors do not match in_features {k}")
        if y is None:
            y = torch.empty((m, n), dtype=out_dtype, device=L.packed.device)
        table[g] = Layer(_dev(L.packed, "packed", (torch.int8,)), _dev(L.s_rel, "s_rel", (torch.uint8,)),
                         _dev(L.s_channel, "s_channel", (torch.float32,)),
                         _dev(L.codebook, "codebook", (torch.float32,)), n,
                         _dev(y, "y", (torch.float32, torch.bfloat16)))
        ys.append(y)
    dt = {_fdtype(y) for y in ys}
    if len(dt) != 1:
        raise ValueError("all outputs of one call must have the same dtype")
    return table, ys, dt.pop()


def linear_multi(x_q: torch.Tensor, s_x: torch.Tensor, layers, out_dtype=torch.float32, outs=None):
    """The product of prepared activations with several layers (one launch at GEMV sizes)."""
    m, k = x_q.shape
    if tuple(s_x.shape) != (m,):
        raise ValueError("s_x must be [M]")
    table, ys, ydt = _layer_table(layers, m, k, out_dtype, outs)
    _check(lib().w4a8_linear_multi(_dev(x_q, "x_q", (torch.int8,)), _dev(s_x, "s_x", (torch.float32,)), m, k,
                                   len(ys), C.addressof(table), ydt, _stream()), "w4a8_linear_multi")
    return ys


def forward_multi(x: torch.Tensor, layers, out_dtype=torch.float32, outs=None, x_q=None, s_x=None):
    """prepare_activation + linear_multi (one launch for the fused decode sizes)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    xp = _dev(x, "x", (torch.float32, torch.bfloat16))
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty((m,), dtype=torch.float32, device=x.device)
    table, ys, ydt = _layer_table(layers, m, k, out_dtype, outs)
    _check(lib().w4a8_forward_multi(xp, _fdtype(x), m, k, len(ys), C.addressof(table), ydt,
                                    _dev(x_q, "x_q", (torch.int8,)), _dev(s_x, "s_x", (torch.float32,)),
                                    _stream()), "w4a8_forward_multi")
    return ys


def linear_pick(m: int, n: int, k: int) -> int:
    return int(lib().w4a8_linear_pick(m, n, k))


# ----------------------------------------------------------------------------- W8A8 comparator

@dataclass
class W8Linear:
    """The int8-weight comparator layer: w_q int8 [N, K] (rotated rows), s_w fp32 [N]."""
    w_q: torch.Tensor
    s_w: torch.Tensor


def w8a8_quantize_weight(w: torch.Tensor) -> W8Linear:
    """Quantise a [N, K] fp32/bf16 weight to per-row int8 of its rotated rows."""
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    wp = _dev(w, "w", (torch.float32, torch.bfloat16))
    w_q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    s_w = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check(lib().w4a8_w8a8_quantize_weight(wp, _fdtype(w), n, k, w_q.data_ptr(), s_w.data_ptr(), _stream()),
           "w4a8_w8a8_quantize_weight")
    return W8Linear(w_q, s_w)


def w8a8_linear(x_q: torch.Tensor, s_x: torch.Tensor, layer: W8Linear, out_dtype=torch.float32,
                algo: int = ALGO_AUTO, out: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] of the W8A8 comparator (algo: ALGO_AUTO, ALGO_GEMV or ALGO_MFMA_I8)."""
    m, k = x_q.shape
    n = layer.w_q.shape[0]
    if tuple(layer.w_q.shape) != (n, k) or tuple(layer.s_w.shape) != (n,) or tuple(s_x.shape) != (m,):
        raise ValueError(f"inconsistent shapes: x_q {tuple(x_q.shape)}, s_x {tuple(s_x.shape)}, "
                         f"w_q {tuple(layer.w_q.shape)}, s_w {tuple(layer.s_w.shape)}")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x_q.device)
    _check(lib().w4a8_w8a8_linear(_dev(x_q, "x_q", (torch.int8,)), _dev(s_x, "s_x", (torch.float32,)), m, k,
                                  _dev(layer.w_q, "w_q", (torch.int8,)), _dev(layer.s_w, "s_w", (torch.float32,)),
                                  n, _dev(out, "y", (torch.float32, torch.bfloat16)), _fdtype(out), algo,
                                  _stream()), "w4a8_w8a8_linear")
    return out
