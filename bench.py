"""Benchmark of the W4A8 codebook linear layer on one MI355X.

Headline (one JSON line on stdout): effective weight GB/s of the decode hot path at M=1.
One step = the whole per-call path for one token on the two MLP shapes of a 27B-class
decoder -- prepare_activation + linear for gate/up (N=17408, K=5120) and for down
(N=5120, K=17408) -- with inputs resident in HBM.  Each shape has 8 distinct weight copies
(~400 MB per shape, beyond the 256 MB Infinity Cache) and consecutive steps use
consecutive copies, so every step streams its weights from HBM.  Steps are replayed from
HIP graphs (8 steps per graph) so host launch cost does not pace the GPU.

value = weight-side bytes per step (packed + group scales + row scales + codebook of both
matrices) / measured time per step.  The same line carries:
  roofline      the decode GEMV kernel: algorithmic bytes per launch / its average launch
                duration (HIP events around back-to-back launches on the launch stream)
                against 8 TB/s;
  prefill       the int8-MFMA GEMM at M=2048 on both shapes: int8 TOPS against 5.0 POPS;
  cpu_baseline  the CPU oracle (prepare + fp64 product) on the same M=1 workload, timed on
                this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
F16_PEAK_TFLOPS = 2500.0
COPIES = 8
METRIC = "W4A8 linear: effective weight GB/s (M=1) + int8 TOPS (M=2048) on 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(n, k):
    return n * k // 2 + n * k // 16 + 4 * n + 64


def gemv_bytes(n, k, m=1):
    """Algorithmic HBM bytes of one linear launch: weights + x_q + s_x + fp32 y."""
    return weight_bytes(n, k) + m * k + 4 * m + 4 * m * n


def build_layers(w, torch, shapes, copies):
    import synthetic as S
    layers = {}
    for (n, k) in shapes:
        W = torch.from_numpy(S.weights(n, k, seed=0)).cuda()
        base = w.quantize_weight(W, seed=0)
        torch.cuda.synchronize()
        del W
        layers[(n, k)] = [w.QuantizedLinear(base.packed.clone(), base.s_rel.clone(),
                                            base.s_channel.clone(), base.codebook.clone())
                          for _ in range(copies)]
        torch.cuda.synchronize()
    return layers


def make_graph(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm: first-call attribute setup happens outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def busy(torch):
    """Keep the GPU busy while the host enqueues what follows (no host-paced gaps)."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(20_000_000)


def time_graph_launches(torch, graph, launches_per_replay, replays):
    """Average GPU time per launch of a graph of back-to-back launches (HIP events on
    the current stream, the stream the library launches on)."""
    busy(torch)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / (launches_per_replay * replays)


def cpu_baseline(shapes, target_s=10.0):
    import oracle as O
    import synthetic as S
    prep = []
    for (n, k) in shapes:
        W = S.weights(n, k, seed=0)
        q = O.quantize_weight(W, seed=0)
        x = S.activations(1, k, seed=0)
        prep.append((n, k, q, x))
    reps, t0 = 0, time.perf_counter()
    while True:
        for (n, k, q, x) in prep:
            xq, sx = O.prepare(x)
            O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    byt = sum(weight_bytes(n, k) for (n, k, _, _) in prep) * reps
    return dict(value=round(byt / el / 1e9, 3), unit="GB/s", cores=O.num_threads(), kind="oracle",
                sample=f"{reps} full M=1 passes (prepare + fp64 product over all rows) of both "
                       f"shapes 17408x5120 and 5120x17408, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic as S
    import w4a8_codebook_gemm_amd as w

    torch.cuda.set_device(0)
    w.lib()
    shapes = [S.MLP_GATE_UP, S.MLP_DOWN]
    layers = build_layers(w, torch, shapes, COPIES)
    xs = {(n, k): torch.from_numpy(S.activations(1, k, seed=0)).cuda() for (n, k) in shapes}
    xqs = {(n, k): (torch.empty((1, k), dtype=torch.int8, device="cuda"),
                    torch.empty((1,), dtype=torch.float32, device="cuda")) for (n, k) in shapes}
    ys = {(n, k): torch.empty((1, n), dtype=torch.float32, device="cuda") for (n, k) in shapes}

    def step(c):
        """The decode hot path for one token on both shapes: rotation + int8 quantisation +
        W4A8 product, fused into one launch per matrix."""
        for sh in shapes:
            w.forward(xs[sh], layers[sh][c], out=ys[sh], x_q=xqs[sh][0], s_x=xqs[sh][1])

    def step_unfused(c):
        for sh in shapes:
            w.prepare_activation(xs[sh], out=xqs[sh])
            w.linear(*xqs[sh], layers[sh][c], out=ys[sh])

    def step_graph(cs, fn=step):
        return make_graph(torch, lambda: [fn(c) for c in cs])

    full = step_graph(range(COPIES))
    rem = args.steps % COPIES
    tail = step_graph(range(rem)) if rem else None

    def run(nsteps):
        for _ in range(nsteps // COPIES):
            full.replay()
        if nsteps % COPIES:
            assert nsteps % COPIES == rem
            tail.replay()

    warm = args.warmup - args.warmup % COPIES
    run(warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / args.steps
    wb = sum(weight_bytes(n, k) for (n, k) in shapes)
    value = wb / (el / args.steps) / 1e9
    log(f"decode step: {ms_step * 1e3:.2f} us, {value:.1f} GB/s effective weight bandwidth")
    unf = step_graph(range(COPIES), step_unfused)
    t_unf = time_graph_launches(torch, unf, COPIES, max(4, args.steps // (4 * COPIES)))
    log(f"decode step with separate prepare launches: {t_unf * 1e6:.2f} us")

    # the dominant kernel: decode GEMV, back-to-back launches over the 16 distinct matrices
    for sh in shapes:
        w.prepare_activation(xs[sh], out=xqs[sh])
    torch.cuda.synchronize()
    gemv_g = make_graph(torch, lambda: [w.linear(*xqs[sh], layers[sh][c], out=ys[sh], algo=w.ALGO_GEMV)
                                        for c in range(COPIES) for sh in shapes])
    launches = COPIES * len(shapes)
    t_gemv = time_graph_launches(torch, gemv_g, launches, max(4, args.steps // (4 * COPIES)))
    per_launch = sum(gemv_bytes(n, k) for (n, k) in shapes) / len(shapes)
    achieved = per_launch / t_gemv / 1e9
    log(f"GEMV: {t_gemv * 1e6:.2f} us per launch (mean of both shapes), {achieved:.1f} GB/s")
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None,
                    kernel="k_gemv<1>", per_launch_bytes=int(per_launch),
                    avg_launch_us=round(t_gemv * 1e6, 3))

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warm, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode M=1: rotate + int8-quantise + W4A8 product (w4a8_forward), "
                               "gate/up 17408x5120 and down 5120x17408, "
                               f"{COPIES} distinct weight copies per shape",
                   "tokens": 1, "weight_bytes_per_step": wb},
        "tokens_per_s": round(1.0 / (el / args.steps), 1),
        "unfused_step_us": round(t_unf * 1e6, 2),
        "roofline": roofline,
    }

    if not args.no_prefill:
        M = 2048
        del layers
        torch.cuda.empty_cache()
        pl = build_layers(w, torch, shapes, 2)
        pre = {}
        for (n, k) in shapes:
            xq, sx = w.prepare_activation(torch.from_numpy(S.activations(M, k, seed=0)).cuda())
            y = torch.empty((M, n), dtype=torch.float32, device="cuda")
            for algo, name in ((w.ALGO_MFMA_I8, "mfma_i8"), (w.ALGO_MFMA_F16, "mfma_f16")):
                g = make_graph(torch, lambda: [w.linear(xq, sx, pl[(n, k)][c], out=y, algo=algo)
                                               for c in range(2)])
                t = time_graph_launches(torch, g, 2, 10)
                tops = 2.0 * M * n * k / t / 1e12
                pre[f"{n}x{k}/{name}"] = dict(algo=name, us=round(t * 1e6, 1), tops=round(tops, 1))
                log(f"prefill {name} M={M} {n}x{k}: {t * 1e6:.1f} us, {tops:.1f} TOPS")
        summary = {}
        for name, peak, unit in (("mfma_i8", INT8_PEAK_TOPS, "TOP/s"), ("mfma_f16", F16_PEAK_TFLOPS, "TFLOP/s")):
            vals = [v["tops"] for v in pre.values() if v["algo"] == name]
            mean = float(np.mean(vals))
            summary[name] = dict(tops=round(mean, 1), roofline=dict(
                bound="mfma", achieved=round(mean, 1), peak=peak, unit=unit, frac=round(mean / peak, 4)))
        out["prefill"] = dict(tokens=M, ops_per_gemm="2*M*N*K", shapes=pre, **summary)

    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(shapes)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
