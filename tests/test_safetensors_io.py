"""Four-tensor safetensors interchange (CPU): bit-exact round trip of oracle-quantised layers,
the dtype census, and rejection of inconsistent layers."""
import os

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
import w4a8_codebook_gemm_amd as w
from w4a8_codebook_gemm_amd import safetensors_io as io


def oracle_qlinear(n, k, seed):
    q = O.quantize_weight(S.weights(n, k, seed=seed), seed=seed)
    return w.QuantizedLinear(torch.from_numpy(q["packed"]), torch.from_numpy(q["s_rel"]),
                             torch.from_numpy(q["s_ch"]), torch.from_numpy(q["cb"]))


def test_round_trip_is_bit_exact_and_audit_counts(tmp_path):
    layers = {"model.layers.1.mlp.down_proj": oracle_qlinear(64, 512, 1),
              "model.layers.1.self_attn.q_proj": oracle_qlinear(96, 256, 2)}
    extra = {"model.embed_tokens.weight": torch.zeros(8, 4, dtype=torch.bfloat16),
             "model.norm.weight": torch.ones(4, dtype=torch.float32)}
    path = os.path.join(tmp_path, "m.safetensors")
    io.save_layers(path, layers, extra, metadata={"quantization": "asym_w4a8_int8"})
    back = io.load_layers(path)
    assert set(back) == set(layers)
    for name, L in layers.items():
        B = back[name]
        assert B.s_rel.dtype == torch.uint8
        for a, b in ((L.packed, B.packed), (L.s_rel, B.s_rel), (L.s_channel, B.s_channel), (L.codebook, B.codebook)):
            assert a.dtype == b.dtype and torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    au = io.audit(path)
    # per quantised layer: one I8, one F8_E4M3 and two F32 (s_channel, codebook); plus extras
    assert au.quantized_layers == 2
    assert au.dtypes == {"BF16": 1, "F32": 2 * 2 + 1, "F8_E4M3": 2, "I8": 2}
    assert au.tensors == 4 * 2 + 2
    assert au.layers["model.layers.1.mlp.down_proj"] == (64, 512)
    assert au.parameters == 64 * 256 + 64 * 32 + 64 + 16 + 96 * 128 + 96 * 16 + 96 + 16 + 32 + 4


def test_stored_s_rel_is_e4m3_with_the_library_bits(tmp_path):
    L = oracle_qlinear(16, 256, 3)
    path = os.path.join(tmp_path, "one.safetensors")
    io.save_layers(path, {"l": L})
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        t = f.get_tensor("l.weight_s_rel")
    assert t.dtype == torch.float8_e4m3fn
    np.testing.assert_array_equal(t.view(torch.uint8).numpy(), L.s_rel.numpy())
    # the stored scales decode to the oracle's e4m3 values
    dec = np.array([O.e4m3_decode(c) for c in L.s_rel.numpy().ravel()], dtype=np.float32)
    np.testing.assert_array_equal(t.float().numpy().ravel(), dec)


def test_inconsistent_layers_are_rejected(tmp_path):
    L = oracle_qlinear(16, 256, 4)
    bad = [w.QuantizedLinear(L.packed[:, :64], L.s_rel, L.s_channel, L.codebook),        # K mismatch
           w.QuantizedLinear(L.packed, L.s_rel, L.s_channel[:8], L.codebook),            # rows
           w.QuantizedLinear(L.packed, L.s_rel, L.s_channel, L.codebook[:8]),            # levels
           w.QuantizedLinear(L.packed.view(torch.uint8), L.s_rel, L.s_channel, L.codebook)]
    for i, B in enumerate(bad):
        with pytest.raises(io.FormatError):
            io.save_layers(os.path.join(tmp_path, f"b{i}.safetensors"), {"l": B})
    # K not a multiple of the rotation block (4304 = 16 x 269 cannot be rotated in 256-blocks)
    odd = w.QuantizedLinear(torch.zeros(2, 2152, dtype=torch.int8), torch.zeros(2, 269, dtype=torch.uint8),
                            torch.ones(2), torch.zeros(16))
    with pytest.raises(io.FormatError):
        io.save_layers(os.path.join(tmp_path, "odd.safetensors"), {"l": odd})


def test_incomplete_layers_are_not_loaded(tmp_path):
    from safetensors.torch import save_file
    path = os.path.join(tmp_path, "partial.safetensors")
    save_file({"a.weight": torch.zeros(2, 128, dtype=torch.int8), "a.weight_codebook": torch.zeros(16)}, path)
    assert io.load_layers(path) == {}
    assert io.audit(path).quantized_layers == 0
