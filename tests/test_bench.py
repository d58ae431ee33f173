"""bench.py's host-side pieces, without a GPU: the algorithmic byte counts that the roofline
figures divide by (against the format's tensor sizes), the committed traffic figure, and the
one-GPU contract."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_weight_bytes_are_the_format_tensors():
    # packed int8 [N][K/2], e4m3 s_rel [N][K/16], fp32 s_channel [N], fp32 codebook [16]
    for n, k in [(17408, 5120), (5120, 17408), (256, 512)]:
        assert bench.weight_bytes(n, k) == n * (k // 2) + n * (k // 16) + 4 * n + 4 * 16
    assert bench.weight_bytes(17408, 5120) == 44_564_480 + 5_570_560 + 69_632 + 64


def test_launch_bytes():
    # the fused gate+up launch: two layers' weights, fp32 x in once, x_q and s_x out once,
    # both layers' fp32 y
    assert bench.multi_forward_bytes(17408, 5120, 2) == 2 * 50_204_736 + 4 * 5120 + 5120 + 4 + 2 * 4 * 17408
    assert bench.multi_forward_bytes(17408, 5120, 2) == 100_574_340
    assert bench.forward_bytes(5120, 17408) == bench.weight_bytes(5120, 17408) + 5 * 17408 + 4 + 4 * 5120
    assert bench.gemv_bytes(17408, 5120) == bench.weight_bytes(17408, 5120) + 5120 + 4 + 4 * 17408
    assert bench.prepare_bytes(2048, 5120) == 2048 * 5120 * 5 + 4 * 2048
    assert bench.w8_gemv_bytes(17408, 5120) == 17408 * 5120 + 4 * 17408 + 5120 + 4 + 4 * 17408


def test_committed_traffic_matches_the_kernel_source():
    t = bench.measured_traffic()
    assert t is not None, "profiles/k_gemv_fused_m1_mlp_traffic.md was taken on another kernel source"
    # within a few per cent of the algorithmic bytes: nothing re-read
    assert 1.0 <= t / bench.multi_forward_bytes(17408, 5120, 2) < 1.02


def test_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
