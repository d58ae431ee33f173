"""Seeded synthetic inputs for the W4A8 codebook linear layer.

This module is the only code that the CPU oracle side and the HIP side share.  It
produces input tensors only (weights and activations with the shapes and value
distributions of the workloads below) and contains none of the method's arithmetic:
no rotation, no scales, no codebook, no quantisation.

Random numbers come from the SplitMix64 generator (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser
constants as published by Vigna), used in counter form: output i of stream s under
seed S is mix(key(S, s) + (i + 1) * GOLDEN).  Uniforms take the top 53 bits plus a
half step, so they lie strictly inside (0, 1); normals use the Box-Muller transform;
Student-t with 4 degrees of freedom is Z / sqrt(chi2_4 / 4) with
chi2_4 = -2 ln(U1 U2).

Workload shapes follow the model cards' description of a 27B-class hybrid decoder
(hidden size 5120, MLP width 17408; page "Qwen3.8-27B ... GGUF (UD Quants)",
architecture notes) and the quantised-layer format (page "Qwen3.8-27B-uncensored-
w4a8-convrot-ComfyUI", section "Format": rotation block 256, group 16).
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_STREAM_STRIDE = 0xD1B54A32D192ED03  # odd constant separating the streams of one seed

# Streams of one seed.
STREAM_WEIGHT = 1
STREAM_ACT = 2
STREAM_OUTLIER = 3


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    base = (int(seed) + int(stream) * _STREAM_STRIDE) & 0xFFFFFFFFFFFFFFFF
    return _mix(np.array([base], dtype=np.uint64))[0]


def u64(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """n raw 64-bit outputs of stream `stream` under `seed`, starting at counter `offset`."""
    key = stream_key(seed, stream)
    i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + i * GOLDEN)


def uniform01(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """n float64 uniforms strictly inside (0, 1)."""
    r = u64(seed, stream, n, offset) >> np.uint64(11)
    return (r.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """n standard normals (float64) by Box-Muller, two per uniform pair."""
    pairs = (n + 1) // 2
    u = uniform01(seed, stream, 2 * pairs, 2 * offset)
    u1, u2 = u[0::2], u[1::2]
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * pairs, dtype=np.float64)
    z[0::2] = rad * np.cos(2.0 * np.pi * u2)
    z[1::2] = rad * np.sin(2.0 * np.pi * u2)
    return z[:n]


def student_t4(seed: int, stream: int, n: int) -> np.ndarray:
    """n Student-t(4) draws: Z / sqrt(chi2_4 / 4) with chi2_4 = -2 ln(U1 U2)."""
    z = normal(seed, stream, n)
    u = uniform01(seed, stream + 1000, 2 * n)
    chi2 = -2.0 * np.log(u[0::2] * u[1::2])
    return z / np.sqrt(chi2 / 4.0)


def weights(n: int, k: int, seed: int = 0, scale: float = 0.02) -> np.ndarray:
    """Weight matrix W [n, k] fp32, Student-t(4) x scale (row-major, out x in)."""
    return (student_t4(seed, STREAM_WEIGHT, n * k) * scale).astype(np.float32).reshape(n, k)


def outlier_channels(k: int, count: int, seed: int = 0) -> np.ndarray:
    """`count` distinct channel indices in [0, k), by a partial Fisher-Yates shuffle."""
    count = min(count, k)
    perm = np.arange(k, dtype=np.int64)
    r = u64(seed, STREAM_OUTLIER, count)
    for i in range(count):
        j = i + int(r[i] % np.uint64(k - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def default_outliers(k: int) -> int:
    """0.1 % of the channels (at least one), the batched workloads' outlier rate."""
    return max(1, int(round(0.001 * k)))


def activations(m: int, k: int, seed: int = 0, n_outliers: int | None = None,
                outlier_scale: float = 20.0) -> np.ndarray:
    """Activations x [m, k] fp32: N(0, 1) with whole outlier columns scaled by 20."""
    if n_outliers is None:
        n_outliers = default_outliers(k)
    x = normal(seed, STREAM_ACT, m * k).reshape(m, k)
    if n_outliers > 0 and m > 0:
        x[:, outlier_channels(k, n_outliers, seed)] *= outlier_scale
    return x.astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even) and return the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# Workload shapes (out rows N, in features K).  Token counts M per workload.
MLP_GATE_UP = (17408, 5120)
MLP_DOWN = (5120, 17408)
ATTN_SQUARE = (5120, 5120)
ATTN_WIDE = (15360, 5120)

WORKLOADS = {
    "tiny": dict(shapes=[(256, 512)], tokens=[4], n_outliers=2, seed=0),
    "decode_m1": dict(shapes=[MLP_GATE_UP, MLP_DOWN], tokens=[1], seed=0),
    "decode_sweep": dict(shapes=[MLP_GATE_UP, MLP_DOWN, ATTN_SQUARE, ATTN_WIDE],
                         tokens=[1, 2, 4, 8, 16, 32, 64], seed=0),
    "prefill_m2048": dict(shapes=[MLP_GATE_UP, MLP_DOWN], tokens=[2048], seed=0),
    "model_62l": dict(layers=62, shapes_per_layer=[MLP_GATE_UP, MLP_GATE_UP, MLP_DOWN]
                      + [ATTN_SQUARE] * 5, tokens=[1], seed=0),
}
