"""safetensors interchange of quantised layers in the four-tensor format.

Model card "Qwen3.8-27B-uncensored-w4a8-convrot-ComfyUI", section "Format": each quantised
layer carries `weight` (int8, packed 4-bit indices, two per byte), `weight_s_rel`
(fp8_e4m3, one scale per 16 values), `weight_s_channel` (fp32, one scale per output row) and
`weight_codebook` (fp32, the 16 levels).  A layer named `P` is stored as the tensors
`P.weight`, `P.weight_s_rel`, `P.weight_s_channel`, `P.weight_codebook`; s_rel is written as
F8_E4M3 with the same bits the library keeps as uint8.

Section "Verification" audits a file by its dtype counts and checks that each layer's
tensors are consistent; `audit` does the same for the four tensors of every layer.

Only the `safetensors` loader is used: it reads tensors and a JSON header and executes
nothing from the file.
"""
from __future__ import annotations

import collections
from dataclasses import dataclass

import torch
from safetensors import safe_open
from safetensors.torch import save_file

from . import QuantizedLinear

SUFFIXES = ("weight", "weight_s_rel", "weight_s_channel", "weight_codebook")
ROTATION_BLOCK = 256  # in_features must be a multiple of the rotation block


class FormatError(ValueError):
    pass


def _check_layer(name: str, packed, s_rel, s_ch, cb) -> tuple[int, int]:
    if packed.dtype != torch.int8 or packed.dim() != 2:
        raise FormatError(f"{name}.weight: expected int8 [N, K/2], got {packed.dtype} {tuple(packed.shape)}")
    n, half_k = packed.shape
    k = 2 * half_k
    if k % ROTATION_BLOCK:
        raise FormatError(f"{name}: in_features {k} is not a multiple of {ROTATION_BLOCK}")
    if s_rel.dtype not in (torch.float8_e4m3fn, torch.uint8) or tuple(s_rel.shape) != (n, k // 16):
        raise FormatError(f"{name}.weight_s_rel: expected fp8_e4m3 [{n}, {k // 16}], got {s_rel.dtype} "
                          f"{tuple(s_rel.shape)}")
    if s_ch.dtype != torch.float32 or tuple(s_ch.shape) != (n,):
        raise FormatError(f"{name}.weight_s_channel: expected fp32 [{n}], got {s_ch.dtype} {tuple(s_ch.shape)}")
    if cb.dtype != torch.float32 or tuple(cb.shape) != (16,):
        raise FormatError(f"{name}.weight_codebook: expected fp32 [16], got {cb.dtype} {tuple(cb.shape)}")
    return n, k


def save_layers(path: str, layers: dict[str, QuantizedLinear], extra: dict[str, torch.Tensor] | None = None,
                metadata: dict[str, str] | None = None) -> None:
    """Write quantised layers (and any extra, unquantised tensors) to one safetensors file."""
    tensors: dict[str, torch.Tensor] = {}
    for name, L in layers.items():
        _check_layer(name, L.packed, L.s_rel, L.s_channel, L.codebook)
        tensors[f"{name}.weight"] = L.packed.detach().contiguous().cpu()
        tensors[f"{name}.weight_s_rel"] = L.s_rel.detach().contiguous().cpu().view(torch.float8_e4m3fn)
        tensors[f"{name}.weight_s_channel"] = L.s_channel.detach().contiguous().cpu()
        tensors[f"{name}.weight_codebook"] = L.codebook.detach().contiguous().cpu()
    for key, t in (extra or {}).items():
        if key in tensors:
            raise FormatError(f"duplicate tensor name {key}")
        tensors[key] = t.detach().contiguous().cpu()
    save_file(tensors, path, metadata=metadata)


def layer_names(keys) -> list[str]:
    """Prefixes P for which all four tensors P.weight* are present."""
    have = set(keys)
    out = []
    for key in sorted(have):
        if key.endswith(".weight_codebook"):
            p = key[: -len(".weight_codebook")]
            if all(f"{p}.{s}" in have for s in SUFFIXES):
                out.append(p)
    return out


def load_layers(path: str, device: str | torch.device = "cpu") -> dict[str, QuantizedLinear]:
    """Read every four-tensor layer of a file (s_rel as the uint8 bits the library uses)."""
    out = {}
    with safe_open(path, framework="pt") as f:
        for p in layer_names(f.keys()):
            packed = f.get_tensor(f"{p}.weight")
            s_rel = f.get_tensor(f"{p}.weight_s_rel")
            s_ch = f.get_tensor(f"{p}.weight_s_channel")
            cb = f.get_tensor(f"{p}.weight_codebook")
            _check_layer(p, packed, s_rel, s_ch, cb)
            if s_rel.dtype == torch.float8_e4m3fn:
                s_rel = s_rel.view(torch.uint8)
            out[p] = QuantizedLinear(packed.to(device), s_rel.to(device), s_ch.to(device), cb.to(device))
    return out


@dataclass
class Audit:
    tensors: int
    parameters: int
    dtypes: dict[str, int]
    quantized_layers: int
    layers: dict[str, tuple[int, int]]   # name -> (out_features, in_features)


def audit(path: str) -> Audit:
    """Dtype census and per-layer consistency of a file; raises FormatError on a bad layer."""
    dtypes: collections.Counter = collections.Counter()
    params = 0
    layers = {}
    with safe_open(path, framework="pt") as f:
        keys = list(f.keys())
        for key in keys:
            sl = f.get_slice(key)
            dtypes[sl.get_dtype()] += 1
            n = 1
            for d in sl.get_shape():
                n *= d
            params += n
        for p in layer_names(keys):
            layers[p] = _check_layer(p, f.get_tensor(f"{p}.weight"), f.get_tensor(f"{p}.weight_s_rel"),
                                     f.get_tensor(f"{p}.weight_s_channel"), f.get_tensor(f"{p}.weight_codebook"))
    return Audit(tensors=len(keys), parameters=params, dtypes=dict(sorted(dtypes.items())),
                 quantized_layers=len(layers), layers=layers)
