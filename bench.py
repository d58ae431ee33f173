"""Benchmark of the W4A8 codebook linear layer on one MI355X.

Headline (one JSON line on stdout): effective weight GB/s of the decode hot path at M=1.
One step = the MLP block of a 27B-class decoder for one token: Hadamard-256 rotation +
per-token int8 quantisation + W4A8 product for gate and up (N=17408, K=5120, one input, one
fused launch: w4a8_forward_multi) and for down (N=5120, K=17408, its own input: w4a8_forward),
with inputs resident in HBM.  There are 8 distinct copies of the block's weights (~1.2 GB,
beyond the 256 MB Infinity Cache) and consecutive steps use consecutive copies, so every step
streams its weights from HBM.  Steps are replayed from HIP graphs (8 steps per graph) so host
launch cost does not pace the GPU.  The nonlinearity between up and down is not part of the
layer; down reads a synthetic input of its own.

value = weight-side bytes per step (packed + group scales + row scales + codebook of the three
matrices) / measured time per step.  The same line carries:
  roofline      the dominant kernel, the fused gate+up launch k_gemv<1,1,8>: algorithmic
                bytes per launch / its average launch duration (HIP events on the launch
                stream around graph replays of that launch) against 8 TB/s; traffic = HBM
                bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a
                copy-kernel calibration, when the committed counter summary matches the
                current kernel source (else null);
  down          the same figures for the fused down launch k_gemv<1,1,1>;
  gemv          the prepared-input GEMV kernel (w4a8_linear, M=1, one layer) on both shapes;
  sweep         batched decode: M in {1,2,4,8,16,32,64} x four projection shapes, every
                kernel that supports the point, plus the automatic choice (prepare included);
  model         62 decoder layers x 8 projections (13.9 GB resident, 496 allocations), one
                token = one fused multi-layer call per input (248 launches) from one HIP graph,
                and the same token with one launch per projection (496);
  prefill       M=2048 GEMMs on both MLP shapes: the int8-codebook and fp16-codebook routes
                (f16 MFMA on decoded weights), the requantised route (int8 MFMA) and the
                int8-codebook product with the per-group fold (int8 MFMA + vector ALU);
  w8a8          the INT8 ConvRot comparator (same rotation and int8 activations, per-row
                int8 weights): decode GEMV on both MLP shapes (prepared x_q), a decode step
                with its prepare launches beside the W4A8 unfused step, and M=2048 GEMMs;
  quantize      offline w4a8_quantize_weight on both MLP shapes from fp32 and bf16 weights
                (rotation, scales, seeded Lloyd-Max fit on 2^20 samples, assignment, packing):
                weights per second, including the fit's fixed cost;
  cpu_baseline  the CPU oracle (prepare + fp64 product) on the same M=1 workload, timed on
                this host's cores.

--pmc-pass runs each kernel a few times eagerly (plus a plain copy of known size for
calibration) and prints nothing else: it is the program profiled by the counter runs.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
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
SWEEP_M = (1, 2, 4, 8, 16, 32, 64)
MODEL_LAYERS = 62
CALIB_BYTES = 1 << 30  # the copy kernel of the counter calibration reads and writes 1 GiB
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemv_fused_m1_mlp_traffic.md")
GEMV_SOURCES = ("w4a8_codebook_gemm_amd/csrc/k_gemv.hip", "w4a8_codebook_gemm_amd/csrc/w4a8_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(n, k):
    return n * k // 2 + n * k // 16 + 4 * n + 64


def gemv_bytes(n, k, m=1):
    """Algorithmic HBM bytes of one prepared-input linear launch: weights + x_q + s_x + fp32 y."""
    return weight_bytes(n, k) + m * k + 4 * m + 4 * m * n


def forward_bytes(n, k, m=1):
    """Algorithmic HBM bytes of one fused forward launch: weights + fp32 x in + x_q, s_x out
    + fp32 y out."""
    return weight_bytes(n, k) + 4 * m * k + m * k + 4 * m + 4 * m * n


def source_sha256(paths=GEMV_SOURCES):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per fused-forward launch from the committed counter summary, or None when it
    is missing or was taken on a different kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch=(\d+)\s+source_sha256=([0-9a-f]{64})", text)
    if not m or m.group(2) != source_sha256():
        return None
    return int(m.group(1))


def build_layers(w, torch, shapes, copies):
    import synthetic as S
    layers = {}
    for (n, k) in shapes:
        W = torch.from_numpy(S.weights(n, k, seed=0)).cuda()
        base = w.quantize_weight(W, seed=0)
        torch.cuda.synchronize()
        del W
        layers[(n, k)] = [clone_layer(w, base) for _ in range(copies)]
        torch.cuda.synchronize()
    return layers


def clone_layer(w, base):
    return w.QuantizedLinear(base.packed.clone(), base.s_rel.clone(), base.s_channel.clone(),
                             base.codebook.clone())


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


PROBES = os.path.join(ROOT, "bench_probes.so")


def probes():
    """The measurement helpers of bench_probes.hip (built by __graft_entry__.build()), or
    None when they are not built."""
    if not os.path.exists(PROBES):
        return None
    lib = ctypes.CDLL(PROBES)
    lib.bench_read_launch.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.bench_read_launch.restype = ctypes.c_int
    lib.bench_stream_launch.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.bench_stream_launch.restype = ctypes.c_int
    return lib


def read_ceiling(torch, nbytes, copies=COPIES):
    """The achievable HBM read rate at nbytes per launch: a plain streaming read (non-temporal
    16-byte loads, each workgroup on a contiguous share) over `copies` distinct buffers, as
    the decode kernels rotate through weight copies, timed like the kernels.  The best over
    workgroup widths 256 / 512 / 1024 threads, 2 / 4 / 8 loads in flight per thread and one or
    two workgroups per compute unit.  Returns (GB/s, config, GB/s of the decode GEMV's own
    launch shape: one 1024-thread workgroup per CU, two loads in flight per lane) or None when
    the helper is not built."""
    lib = probes()
    if lib is None:
        return None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = nbytes // 16 * 16
    bufs = [torch.full((n,), c + 1, dtype=torch.uint8, device="cuda") for c in range(copies)]
    sink = torch.zeros(2 * cus * 1024, dtype=torch.int32, device="cuda")
    best, cfg, own = 0.0, None, None
    for per_cu in (1, 2):
        for threads in (256, 512, 1024):
            for depth in (2, 4, 8):
                blocks = per_cu * cus

                def launch():
                    st = torch.cuda.current_stream().cuda_stream
                    for b in bufs:
                        rc = lib.bench_read_launch(b.data_ptr(), n, sink.data_ptr(), blocks, threads, depth, st)
                        if rc != 0:
                            raise RuntimeError(f"bench_read_launch: HIP error {rc}")
                g = make_graph(torch, launch)
                t = time_kernel_graph(torch, g) / copies
                if (per_cu, threads, depth) == (1, 1024, 2):
                    own = n / t / 1e9
                if n / t / 1e9 > best:
                    best, cfg = n / t / 1e9, dict(workgroups_per_cu=per_cu, threads=threads,
                                                  loads_in_flight_per_thread=depth,
                                                  kib_in_flight_per_cu=per_cu * threads * depth * 16 // 1024,
                                                  us_per_launch=round(t * 1e6, 3))
                del g
    del bufs
    torch.cuda.empty_cache()
    return best, cfg, own


def stream_ceiling(torch, in_bytes, copies=COPIES):
    """The achievable rate of a streaming read + write in the activation preparation's
    proportion (4 bytes read per byte written, fp32 in and int8 out) at in_bytes read per
    launch, over `copies` distinct inputs, timed like the kernels: the best over one, two or
    four workgroups per compute unit, 256 / 512 / 1024 threads and 1 / 2 / 4 loads in flight
    per thread.  Returns (GB/s of read + written bytes, config) or None when the helper is not
    built."""
    lib = probes()
    if lib is None:
        return None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = in_bytes // 16 * 16
    srcs = [torch.full((n,), c + 1, dtype=torch.uint8, device="cuda") for c in range(copies)]
    dst = torch.empty((n // 4,), dtype=torch.uint8, device="cuda")
    best, cfg = 0.0, None
    for per_cu in (1, 2, 4):
        for threads in (256, 512, 1024):
            for depth in (1, 2, 4):
                blocks = per_cu * cus

                def launch():
                    st = torch.cuda.current_stream().cuda_stream
                    for b in srcs:
                        rc = lib.bench_stream_launch(b.data_ptr(), n, dst.data_ptr(), blocks, threads, depth, st)
                        if rc != 0:
                            raise RuntimeError(f"bench_stream_launch: HIP error {rc}")
                g = make_graph(torch, launch)
                t = time_kernel_graph(torch, g) / copies
                rate = (n + n // 4) / t / 1e9
                if rate > best:
                    best, cfg = rate, dict(workgroups_per_cu=per_cu, threads=threads, loads_in_flight_per_thread=depth,
                                           us_per_launch=round(t * 1e6, 3))
                del g
    del srcs, dst
    torch.cuda.empty_cache()
    return best, cfg


def busy(torch):
    """Keep the GPU busy while the host enqueues what follows (no host-paced gaps)."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(20_000_000)


def time_kernel_graph(torch, graph, replays=4, bursts=5):
    """Per-kernel figures: the median over `bursts` short runs of `replays` graph replays, each
    after the busy-wait.  A memory-bound launch sustained for milliseconds slows down by up to
    about 12% (the power draw of a full-bandwidth stream); the headline step and the model are
    timed sustained, the per-kernel rooflines in short runs, which is what a kernel trace of
    the same launches records."""
    ts = sorted(time_graph(torch, graph, replays) for _ in range(bursts))
    return ts[len(ts) // 2]


def time_graph(torch, graph, replays):
    """GPU seconds per replay of a graph (HIP events on the current stream, the stream the
    graph and the library's kernels run on)."""
    busy(torch)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / replays


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
    # prefill beside it: the fp64 product of 256 rows x 2048 tokens of the gate/up shape (a
    # slice of the M = 2048 GEMM, whose cost scales linearly with the rows)
    n, k, q, _ = prep[0]
    xq, sx = O.prepare(S.activations(2048, k, seed=0))
    rows = np.arange(256)
    t1 = time.perf_counter()
    O.linear_ref(xq, sx, q["packed"], q["s_rel"], q["s_ch"], q["cb"], rows, None)
    tp = time.perf_counter() - t1
    return dict(value=round(byt / el / 1e9, 3), unit="GB/s", cores=O.num_threads(), kind="oracle",
                sample=f"{reps} full M=1 passes (prepare + fp64 product over all rows) of both "
                       f"shapes 17408x5120 and 5120x17408, {el:.1f} s",
                prefill_gops=round(2.0 * 2048 * 256 * k / tp / 1e9, 2),
                prefill_sample=f"fp64 product of 256 of the {n} rows x 2048 tokens at K = {k}, {tp:.2f} s "
                               f"(the full GEMM would take {tp * n / 256:.0f} s)")


def mlp_layers(w, torch, S, copies):
    """`copies` distinct MLP blocks of the 27B-class shape: gate and up 17408x5120, down
    5120x17408 (each block's weights are its own allocations, so nothing stays cached)."""
    gu, dn = S.MLP_GATE_UP, S.MLP_DOWN
    L = build_layers(w, torch, [gu, dn], 2 * copies)
    return [dict(gate=L[gu][2 * c], up=L[gu][2 * c + 1], down=L[dn][c]) for c in range(copies)]


def multi_forward_bytes(n, k, g, m=1):
    """Algorithmic HBM bytes of one fused multi-layer forward launch over g layers of n x k:
    the weights, fp32 x in once, x_q and s_x out once, fp32 y of every layer."""
    return g * weight_bytes(n, k) + 4 * m * k + m * k + 4 * m + 4 * m * n * g


def decode(w, torch, S, args, shapes):
    """The headline: one decode step of the MLP block at M=1 -- gate and up in one fused launch
    (w4a8_forward_multi: rotate + quantise the MLP input, then both products), down in a second
    (w4a8_forward on its own input) -- plus the per-kernel rooflines."""
    (ng, kg), (nd, kd) = S.MLP_GATE_UP, S.MLP_DOWN
    blocks = mlp_layers(w, torch, S, COPIES)
    x_in = torch.from_numpy(S.activations(1, kg, seed=0)).cuda()
    x_hid = torch.from_numpy(S.activations(1, kd, seed=1)).cuda()
    xq_in = (torch.empty((1, kg), dtype=torch.int8, device="cuda"), torch.empty((1,), dtype=torch.float32, device="cuda"))
    xq_hid = (torch.empty((1, kd), dtype=torch.int8, device="cuda"), torch.empty((1,), dtype=torch.float32, device="cuda"))
    y_gu = [torch.empty((1, ng), dtype=torch.float32, device="cuda") for _ in range(2)]
    y_dn = torch.empty((1, nd), dtype=torch.float32, device="cuda")

    def gate_up(c):
        b = blocks[c]
        w.forward_multi(x_in, [b["gate"], b["up"]], outs=y_gu, x_q=xq_in[0], s_x=xq_in[1])

    def down(c):
        w.forward(x_hid, blocks[c]["down"], out=y_dn, x_q=xq_hid[0], s_x=xq_hid[1])

    def step(c):
        gate_up(c)
        down(c)

    def step_unfused(c):
        b = blocks[c]
        w.prepare_activation(x_in, out=xq_in)
        w.linear_multi(*xq_in, [b["gate"], b["up"]], outs=y_gu)
        w.prepare_activation(x_hid, out=xq_hid)
        w.linear(*xq_hid, b["down"], out=y_dn)

    full = make_graph(torch, lambda: [step(c) for c in range(COPIES)])
    tails = {r: make_graph(torch, lambda: [step(c) for c in range(r)])
             for r in {args.steps % COPIES, args.warmup % COPIES} if r}

    def run(nsteps):
        """Exactly nsteps steps: whole graphs of COPIES steps, then a graph of the rest."""
        for _ in range(nsteps // COPIES):
            full.replay()
        if nsteps % COPIES:
            tails[nsteps % COPIES].replay()

    warm = args.warmup
    run(warm)
    torch.cuda.synchronize()
    busy(torch)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    run(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    el = ev0.elapsed_time(ev1) * 1e-3
    ms_step = el * 1e3 / args.steps
    wb = 2 * weight_bytes(ng, kg) + weight_bytes(nd, kd)
    value = wb / (el / args.steps) / 1e9
    log(f"decode step (MLP block): {ms_step * 1e3:.2f} us, {value:.1f} GB/s effective weight bandwidth "
        f"(host wall clock incl. the busy-wait kernel {wall:.3f} s)")

    # the dominant kernel: the fused gate+up launch (two thirds of the step's bytes), timed in a
    # graph of its own launches; the down launch beside it
    reps = max(4, args.steps // (4 * COPIES))
    g_gu = make_graph(torch, lambda: [gate_up(c) for c in range(COPIES)])
    t_gu = time_kernel_graph(torch, g_gu) / COPIES
    t_gu_sustained = time_graph(torch, g_gu, reps) / COPIES
    g_dn = make_graph(torch, lambda: [down(c) for c in range(COPIES)])
    t_dn = time_kernel_graph(torch, g_dn) / COPIES
    per_gu = multi_forward_bytes(ng, kg, 2)
    per_dn = forward_bytes(nd, kd)
    ach = per_gu / t_gu / 1e9
    traffic = measured_traffic()
    roofline = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel="k_gemv<1,1,8> (fused rotate + quantise + W4A8 GEMV of gate and up, fp32 x)",
                    per_launch_bytes=int(per_gu), avg_launch_us=round(t_gu * 1e6, 3),
                    avg_launch_us_sustained=round(t_gu_sustained * 1e6, 3))
    rcc = read_ceiling(torch, int(per_gu))
    if rcc:
        rc, cfg, own = rcc
        roofline["read_ceiling_gbs"] = round(rc, 1)
        roofline["read_ceiling_config"] = cfg
        roofline["frac_of_read_ceiling"] = round(ach / rc, 4)
        # the same plain read in the kernel's own launch shape: what its fixed costs are measured against
        roofline["read_same_shape_gbs"] = round(own, 1)
        roofline["frac_of_read_same_shape"] = round(ach / own, 4)
        log(f"plain read of {per_gu / 1e6:.1f} MB per launch: {rc:.1f} GB/s ({cfg}); the fused gate+up "
            f"launch reaches {ach / rc * 100:.1f}% of it")
    down_k = dict(kernel="k_gemv<1,1,1> (fused rotate + quantise + W4A8 GEMV of down, fp32 x)",
                  avg_launch_us=round(t_dn * 1e6, 3), per_launch_bytes=int(per_dn),
                  achieved=round(per_dn / t_dn / 1e9, 1), frac=round(per_dn / t_dn / 1e9 / HBM_PEAK_GBS, 4))
    log(f"fused gate+up: {t_gu * 1e6:.2f} us per launch, {ach:.1f} GB/s algorithmic, traffic {traffic}; "
        f"fused down: {t_dn * 1e6:.2f} us, {per_dn / t_dn / 1e9:.1f} GB/s")

    unf = make_graph(torch, lambda: [step_unfused(c) for c in range(COPIES)])
    t_unf = time_graph(torch, unf, reps) / COPIES
    log(f"decode step with separate prepare launches: {t_unf * 1e6:.2f} us")

    # the single-layer GEMV on prepared activations, both MLP shapes
    w.prepare_activation(x_in, out=xq_in)
    w.prepare_activation(x_hid, out=xq_hid)
    torch.cuda.synchronize()
    gemv_g = make_graph(torch, lambda: [(w.linear(*xq_in, blocks[c]["gate"], out=y_gu[0], algo=w.ALGO_GEMV),
                                         w.linear(*xq_hid, blocks[c]["down"], out=y_dn, algo=w.ALGO_GEMV))
                                        for c in range(COPIES)])
    t_gemv = time_kernel_graph(torch, gemv_g) / (COPIES * 2)
    per_gemv = (gemv_bytes(ng, kg) + gemv_bytes(nd, kd)) / 2
    log(f"GEMV (prepared x_q): {t_gemv * 1e6:.2f} us per launch, {per_gemv / t_gemv / 1e9:.1f} GB/s")
    gemv = dict(kernel="k_gemv<1,0,1> (prepared int8 x, one layer)", avg_launch_us=round(t_gemv * 1e6, 3),
                per_launch_bytes=int(per_gemv), achieved=round(per_gemv / t_gemv / 1e9, 1),
                frac=round(per_gemv / t_gemv / 1e9 / HBM_PEAK_GBS, 4))
    out = dict(value=value, ms_step=ms_step, warm=warm, wb=wb, roofline=roofline, gemv=gemv, down=down_k,
               unfused_step_us=round(t_unf * 1e6, 2), tokens_per_s=round(1.0 / (el / args.steps), 1))
    del blocks
    return out


def sweep(w, torch, S):
    """Batched decode: every kernel that supports (M, shape), the K-split skinny kernel of
    w4a8_linear_ws where it applies, and the automatic choice of w4a8_forward."""
    shapes = [S.MLP_GATE_UP, S.MLP_DOWN, S.ATTN_SQUARE, S.ATTN_WIDE]
    layers = build_layers(w, torch, shapes, COPIES)
    algos = (("gemv", w.ALGO_GEMV), ("mfma_skinny", w.ALGO_MFMA_SKINNY), ("mfma_i8", w.ALGO_MFMA_I8),
             ("mfma_f16", w.ALGO_MFMA_F16))
    res = {}
    for (n, k) in shapes:
        for m in SWEEP_M:
            x = torch.from_numpy(S.activations(m, k, seed=0)).cuda()
            xq, sx = w.prepare_activation(x)
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            point = {}
            for name, algo in algos:
                try:  # the warm call (before capture) rejects points outside a kernel's range
                    g = make_graph(torch, lambda: [w.linear(xq, sx, layers[(n, k)][c], out=y, algo=algo)
                                                   for c in range(COPIES)])
                except w.W4A8Error as e:
                    if e.status != 2:
                        raise
                    continue
                point[name] = round(time_kernel_graph(torch, g) / COPIES * 1e6, 2)
            ws = w.linear_workspace(m, n, k)  # the K-split batched decode (one workspace: calls run in order)
            if ws is not None:
                g = make_graph(torch, lambda: [w.linear_ws(xq, sx, layers[(n, k)][c], ws, out=y)
                                               for c in range(COPIES)])
                point["mfma_skinny_split"] = round(time_kernel_graph(torch, g) / COPIES * 1e6, 2)
            g = make_graph(torch, lambda: [w.forward(x, layers[(n, k)][c], out=y, x_q=xq, s_x=sx)
                                           for c in range(COPIES)])
            t_auto = time_kernel_graph(torch, g) / COPIES
            best = min(point, key=point.get)
            tb = point[best] * 1e-6
            res[f"{n}x{k}/M={m}"] = dict(
                us=point, best=best, auto=w.linear_pick(m, n, k), auto_forward_us=round(t_auto * 1e6, 2),
                weight_gbs=round(weight_bytes(n, k) / tb / 1e9, 1), tokens_per_s=round(m / tb, 1),
                tops=round(2.0 * m * n * k / tb / 1e12, 2))
            log(f"sweep {n}x{k} M={m}: {point} auto(forward) {t_auto * 1e6:.2f} us")
    del layers
    return res


def model(w, torch, S, tokens=20):
    """62 layers x (gate, up 17408x5120; down 5120x17408; five 5120x5120): one token reads every
    weight once.  Inputs per layer: the attention input feeds four square projections, the
    attention output the fifth; the MLP input feeds gate and up; the MLP hidden feeds down.
    Each input is one fused call: w4a8_forward_multi over the layers that read it (4 launches
    per layer).  For comparison, the same token with one launch per projection: the fused
    forward for the first projection of each input, w4a8_linear on its x_q for the others."""
    base = {}
    for sh in (S.MLP_GATE_UP, S.MLP_DOWN, S.ATTN_SQUARE):
        W = torch.from_numpy(S.weights(*sh, seed=0)).cuda()
        base[sh] = w.quantize_weight(W, seed=0)
        torch.cuda.synchronize()
        del W
    layers = []
    for _ in range(MODEL_LAYERS):
        layers.append(dict(attn=[clone_layer(w, base[S.ATTN_SQUARE]) for _ in range(5)],
                           gate=clone_layer(w, base[S.MLP_GATE_UP]), up=clone_layer(w, base[S.MLP_GATE_UP]),
                           down=clone_layer(w, base[S.MLP_DOWN])))
    torch.cuda.synchronize()
    total = sum(weight_bytes(*t) for t in [S.ATTN_SQUARE] * 5 + [S.MLP_GATE_UP] * 2 + [S.MLP_DOWN]) * MODEL_LAYERS
    d, f = S.ATTN_SQUARE[1], S.MLP_DOWN[1]
    xs = {key: torch.from_numpy(S.activations(1, k, seed=i)).cuda()
          for i, (key, k) in enumerate((("attn_in", d), ("attn_out", d), ("mlp_in", d), ("mlp_hid", f)))}
    xq = {key: (torch.empty((1, v.shape[1]), dtype=torch.int8, device="cuda"),
                torch.empty((1,), dtype=torch.float32, device="cuda")) for key, v in xs.items()}
    y5, y17 = (torch.empty((1, n), dtype=torch.float32, device="cuda") for n in (d, S.MLP_GATE_UP[0]))

    y5s = [torch.empty((1, d), dtype=torch.float32, device="cuda") for _ in range(4)]
    y17s = [torch.empty((1, S.MLP_GATE_UP[0]), dtype=torch.float32, device="cuda") for _ in range(2)]

    def token():
        for L in layers:
            w.forward_multi(xs["attn_in"], L["attn"][:4], outs=y5s, x_q=xq["attn_in"][0], s_x=xq["attn_in"][1])
            w.forward(xs["attn_out"], L["attn"][4], out=y5, x_q=xq["attn_out"][0], s_x=xq["attn_out"][1])
            w.forward_multi(xs["mlp_in"], [L["gate"], L["up"]], outs=y17s, x_q=xq["mlp_in"][0],
                            s_x=xq["mlp_in"][1])
            w.forward(xs["mlp_hid"], L["down"], out=y5, x_q=xq["mlp_hid"][0], s_x=xq["mlp_hid"][1])

    def token_separate():
        for L in layers:
            w.forward(xs["attn_in"], L["attn"][0], out=y5, x_q=xq["attn_in"][0], s_x=xq["attn_in"][1])
            for j in (1, 2, 3):
                w.linear(*xq["attn_in"], L["attn"][j], out=y5)
            w.forward(xs["attn_out"], L["attn"][4], out=y5, x_q=xq["attn_out"][0], s_x=xq["attn_out"][1])
            w.forward(xs["mlp_in"], L["gate"], out=y17, x_q=xq["mlp_in"][0], s_x=xq["mlp_in"][1])
            w.linear(*xq["mlp_in"], L["up"], out=y17)
            w.forward(xs["mlp_hid"], L["down"], out=y5, x_q=xq["mlp_hid"][0], s_x=xq["mlp_hid"][1])

    res = {}
    for name, fn in (("multi", token), ("separate", token_separate)):
        g = make_graph(torch, fn)
        g.replay()
        torch.cuda.synchronize()
        res[name] = time_graph(torch, g, tokens)
        del g
    t, t_sep = res["multi"], res["separate"]
    log(f"model: {MODEL_LAYERS} layers, {total / 1e9:.2f} GB, {t * 1e3:.3f} ms/token, "
        f"{1 / t:.1f} tokens/s, {total / t / 1e9:.1f} GB/s (one launch per projection: "
        f"{t_sep * 1e3:.3f} ms/token, {1 / t_sep:.1f} tokens/s)")
    out = dict(layers=MODEL_LAYERS, projections_per_layer=8, launches_per_token=4 * MODEL_LAYERS,
               weight_bytes=total, ms_per_token=round(t * 1e3, 4), tokens_per_s=round(1 / t, 1),
               weight_gbs=round(total / t / 1e9, 1), hbm_bound_tokens_per_s=round(HBM_PEAK_GBS * 1e9 / total, 1),
               one_launch_per_projection=dict(launches_per_token=8 * MODEL_LAYERS, ms_per_token=round(t_sep * 1e3, 4),
                                              tokens_per_s=round(1 / t_sep, 1)))
    del layers, base
    return out


def prefill(w, torch, S, shapes, M=2048):
    pl = build_layers(w, torch, shapes, 2)
    pre = {}
    for (n, k) in shapes:
        xq, sx = w.prepare_activation(torch.from_numpy(S.activations(M, k, seed=0)).cuda())
        y = torch.empty((M, n), dtype=torch.float32, device="cuda")
        for algo, name in ((w.ALGO_MFMA_I8, "mfma_i8"), (w.ALGO_MFMA_F16, "mfma_f16"), (w.ALGO_MFMA_RQ, "mfma_rq"),
                           (w.ALGO_MFMA_I8_FOLD, "mfma_i8_fold")):
            g = make_graph(torch, lambda: [w.linear(xq, sx, pl[(n, k)][c], out=y, algo=algo) for c in range(2)])
            t = time_graph(torch, g, 10) / 2
            tops = 2.0 * M * n * k / t / 1e12
            pre[f"{n}x{k}/{name}"] = dict(algo=name, us=round(t * 1e6, 1), tops=round(tops, 1))
            log(f"prefill {name} M={M} {n}x{k}: {t * 1e6:.1f} us, {tops:.1f} TOPS")
    summary = {}
    # each route against the peak of the matrix-core instruction it runs: the two
    # decoded-weight routes on v_mfma_f32_32x32x16_f16 (the int8 route's int8 x int8 products
    # are exact there), the requantised route on v_mfma_i32_32x32x32_i8
    for name, peak, unit, inst in (("mfma_i8", F16_PEAK_TFLOPS, "TOP/s", "f16"), ("mfma_f16", F16_PEAK_TFLOPS, "TFLOP/s", "f16"),
                                   ("mfma_rq", INT8_PEAK_TOPS, "TOP/s", "i8"), ("mfma_i8_fold", INT8_PEAK_TOPS, "TOP/s", "i8")):
        mean = float(np.mean([v["tops"] for v in pre.values() if v["algo"] == name]))
        summary[name] = dict(tops=round(mean, 1), mfma=inst, roofline=dict(
            bound="mfma", achieved=round(mean, 1), peak=peak, unit=unit, frac=round(mean / peak, 4)))
    del pl
    torch.cuda.empty_cache()
    return dict(tokens=M, ops_per_gemm="2*M*N*K", shapes=pre, prepare=prepare_rate(w, torch, S, M), **summary)


def prepare_bytes(m, k, in_bytes=4):
    """Algorithmic HBM bytes of one activation-preparation launch: x in, x_q and s_x out."""
    return m * k * in_bytes + m * k + 4 * m


def prepare_rate(w, torch, S, M, ks=(5120, 17408)):
    """The activation preparation (k_prepare: rotation + per-token int8) at prefill size, fp32
    input, over COPIES distinct input buffers (larger in all than the Infinity Cache), timed
    like the decode kernels; HBM-bound: 5 K + 4 bytes per token."""
    res = {}
    for k in ks:
        xs = [torch.from_numpy(S.activations(M, k, seed=c)).cuda() for c in range(COPIES)]
        x_q = torch.empty((M, k), dtype=torch.int8, device="cuda")
        s_x = torch.empty((M,), dtype=torch.float32, device="cuda")
        g = make_graph(torch, lambda: [w.prepare_activation(x, out=(x_q, s_x)) for x in xs])
        t = time_kernel_graph(torch, g) / COPIES
        byt = prepare_bytes(M, k)
        del xs, g
        torch.cuda.empty_cache()
        line = dict(kernel="k_prepare_tokens (fp32 x)", us=round(t * 1e6, 2), per_launch_bytes=byt,
                    roofline=dict(bound="hbm", achieved=round(byt / t / 1e9, 1), peak=HBM_PEAK_GBS,
                                  unit="GB/s", frac=round(byt / t / 1e9 / HBM_PEAK_GBS, 4)))
        sc = stream_ceiling(torch, M * k * 4)
        if sc is not None:
            line["roofline"]["stream_ceiling_gbs"] = round(sc[0], 1)
            line["roofline"]["stream_ceiling_config"] = sc[1]
            line["roofline"]["frac_of_stream_ceiling"] = round(byt / t / 1e9 / sc[0], 4)
        res[f"{M}x{k}"] = line
        log(f"prepare M={M} K={k}: {t * 1e6:.2f} us, {byt / t / 1e9:.1f} GB/s"
            + (f"; streaming read + write ceiling {sc[0]:.1f} GB/s ({sc[1]})" if sc else ""))
    return res


def quantize_rate(w, torch, S, shapes, reps=3):
    """Offline quantisation throughput: each call rotates, fits and packs one whole matrix
    (the sort and the strictly ordered fp64 prefix sum of the fit are a fixed cost per call)."""
    res = {}
    for (n, k) in shapes:
        W32 = torch.from_numpy(S.weights(n, k, seed=0)).cuda()
        for name, W in (("f32", W32), ("bf16", W32.to(torch.bfloat16))):
            ws = torch.empty((w.quantize_weight_workspace(n, k),), dtype=torch.uint8, device="cuda")
            w.quantize_weight(W, seed=0, workspace=ws)  # warm
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                w.quantize_weight(W, seed=0, workspace=ws)
            torch.cuda.synchronize()
            t = (time.perf_counter() - t0) / reps
            res[f"{n}x{k}/{name}"] = dict(ms=round(t * 1e3, 2), gweights_per_s=round(n * k / t / 1e9, 2),
                                          input_gbs=round(n * k * W.element_size() / t / 1e9, 1))
            log(f"quantize {n}x{k} {name}: {t * 1e3:.2f} ms, {n * k / t / 1e9:.2f} G weights/s")
        del W32
    return res


def w8_gemv_bytes(n, k, m=1):
    """Algorithmic HBM bytes of one W8A8 linear launch: int8 weights + row scales + x_q + s_x
    + fp32 y."""
    return n * k + 4 * n + m * k + 4 * m + 4 * m * n


def w8a8(w, torch, S, shapes, w4_gemv, w4_unfused_us, w4_prefill, M=2048):
    """The comparator on the same workloads: what the halved weight stream buys on MI355X."""
    layers = {}
    for (n, k) in shapes:
        W = torch.from_numpy(S.weights(n, k, seed=0)).cuda()
        base = w.w8a8_quantize_weight(W)
        torch.cuda.synchronize()
        del W
        layers[(n, k)] = [w.W8Linear(base.w_q.clone(), base.s_w.clone()) for _ in range(COPIES)]
    torch.cuda.synchronize()
    xs = {(n, k): torch.from_numpy(S.activations(1, k, seed=0)).cuda() for (n, k) in shapes}
    xqs = {sh: w.prepare_activation(xs[sh]) for sh in shapes}
    ys = {(n, k): torch.empty((1, n), dtype=torch.float32, device="cuda") for (n, k) in shapes}
    g = make_graph(torch, lambda: [w.w8a8_linear(*xqs[sh], layers[sh][c], out=ys[sh], algo=w.ALGO_GEMV)
                                   for c in range(COPIES) for sh in shapes])
    t_gemv = time_kernel_graph(torch, g) / (COPIES * len(shapes))
    per = sum(w8_gemv_bytes(n, k) for (n, k) in shapes) / len(shapes)

    def step(c):
        for sh in shapes:
            w.prepare_activation(xs[sh], out=xqs[sh])
            w.w8a8_linear(*xqs[sh], layers[sh][c], out=ys[sh])

    g = make_graph(torch, lambda: [step(c) for c in range(COPIES)])
    t_step = time_graph(torch, g, 25) / COPIES
    log(f"W8A8 GEMV: {t_gemv * 1e6:.2f} us per launch, {per / t_gemv / 1e9:.1f} GB/s; decode step "
        f"{t_step * 1e6:.2f} us (W4A8 unfused {w4_unfused_us:.2f} us)")
    out = dict(gemv=dict(kernel="k_w8_gemv<1>", avg_launch_us=round(t_gemv * 1e6, 3), per_launch_bytes=int(per),
                         achieved=round(per / t_gemv / 1e9, 1), frac=round(per / t_gemv / 1e9 / HBM_PEAK_GBS, 4)),
               decode_step_us=round(t_step * 1e6, 2), w4a8_unfused_step_us=w4_unfused_us,
               w4a8_over_w8a8_gemv_time=round(w4_gemv["avg_launch_us"] / (t_gemv * 1e6), 3))
    pre = {}
    for (n, k) in shapes:
        xq, sx = w.prepare_activation(torch.from_numpy(S.activations(M, k, seed=0)).cuda())
        y = torch.empty((M, n), dtype=torch.float32, device="cuda")
        g = make_graph(torch, lambda: [w.w8a8_linear(xq, sx, layers[(n, k)][c], out=y, algo=w.ALGO_MFMA_I8)
                                       for c in range(2)])
        t = time_graph(torch, g, 10) / 2
        tops = 2.0 * M * n * k / t / 1e12
        pre[f"{n}x{k}"] = dict(us=round(t * 1e6, 1), tops=round(tops, 1))
        log(f"W8A8 prefill M={M} {n}x{k}: {t * 1e6:.1f} us, {tops:.1f} TOPS")
    mean = float(np.mean([v["tops"] for v in pre.values()]))
    out["prefill"] = dict(tokens=M, shapes=pre, tops=round(mean, 1), roofline=dict(
        bound="mfma", achieved=round(mean, 1), peak=INT8_PEAK_TOPS, unit="TOP/s", frac=round(mean / INT8_PEAK_TOPS, 4)))
    if w4_prefill:
        best = max(("mfma_i8", "mfma_f16", "mfma_rq"), key=lambda r: w4_prefill[r]["tops"])
        out["prefill"]["w4a8_best_tops"] = w4_prefill[best]["tops"]
        out["prefill"]["w4a8_best_route"] = best
    del layers
    torch.cuda.empty_cache()
    out["model"] = w8a8_model(w, torch, S)
    return out


def w8a8_model(w, torch, S, tokens=10):
    """The 62-layer decoder of `model` with W8A8 weights: one token = prepare each input once,
    then one W8A8 GEMV per projection (496 launches), weights read once per token."""
    base = {}
    for sh in (S.MLP_GATE_UP, S.MLP_DOWN, S.ATTN_SQUARE):
        W = torch.from_numpy(S.weights(*sh, seed=0)).cuda()
        base[sh] = w.w8a8_quantize_weight(W)
        torch.cuda.synchronize()
        del W
    clone = lambda L: w.W8Linear(L.w_q.clone(), L.s_w.clone())
    layers = [dict(attn=[clone(base[S.ATTN_SQUARE]) for _ in range(5)], gate=clone(base[S.MLP_GATE_UP]),
                   up=clone(base[S.MLP_GATE_UP]), down=clone(base[S.MLP_DOWN])) for _ in range(MODEL_LAYERS)]
    torch.cuda.synchronize()
    per_layer = sum(n * k + 4 * n for (n, k) in [S.ATTN_SQUARE] * 5 + [S.MLP_GATE_UP] * 2 + [S.MLP_DOWN])
    total = per_layer * MODEL_LAYERS
    d, f = S.ATTN_SQUARE[1], S.MLP_DOWN[1]
    xs = {key: torch.from_numpy(S.activations(1, k, seed=i)).cuda()
          for i, (key, k) in enumerate((("attn_in", d), ("attn_out", d), ("mlp_in", d), ("mlp_hid", f)))}
    xq = {key: (torch.empty((1, v.shape[1]), dtype=torch.int8, device="cuda"),
                torch.empty((1,), dtype=torch.float32, device="cuda")) for key, v in xs.items()}
    y5, y17 = (torch.empty((1, n), dtype=torch.float32, device="cuda") for n in (d, S.MLP_GATE_UP[0]))

    def token():
        for L in layers:
            w.prepare_activation(xs["attn_in"], out=xq["attn_in"])
            for j in range(4):
                w.w8a8_linear(*xq["attn_in"], L["attn"][j], out=y5)
            w.prepare_activation(xs["attn_out"], out=xq["attn_out"])
            w.w8a8_linear(*xq["attn_out"], L["attn"][4], out=y5)
            w.prepare_activation(xs["mlp_in"], out=xq["mlp_in"])
            w.w8a8_linear(*xq["mlp_in"], L["gate"], out=y17)
            w.w8a8_linear(*xq["mlp_in"], L["up"], out=y17)
            w.prepare_activation(xs["mlp_hid"], out=xq["mlp_hid"])
            w.w8a8_linear(*xq["mlp_hid"], L["down"], out=y5)

    g = make_graph(torch, token)
    g.replay()
    torch.cuda.synchronize()
    t = time_graph(torch, g, tokens)
    log(f"W8A8 model: {MODEL_LAYERS} layers, {total / 1e9:.2f} GB, {t * 1e3:.3f} ms/token, {1 / t:.1f} tokens/s, "
        f"{total / t / 1e9:.1f} GB/s")
    out = dict(weight_bytes=total, launches_per_token=12 * MODEL_LAYERS, ms_per_token=round(t * 1e3, 4),
               tokens_per_s=round(1 / t, 1), weight_gbs=round(total / t / 1e9, 1),
               hbm_bound_tokens_per_s=round(HBM_PEAK_GBS * 1e9 / total, 1))
    del layers, base, g
    return out


def pmc_pass(w, torch, S, shapes):
    """Eager launches for the counter runs: a plain elementwise copy of CALIB_BYTES (reads and
    writes that many bytes once) for calibration, then the MLP block's fused launches (gate+up,
    down) and the prepared-input GEMV on every weight copy, then the prefill GEMMs (three W4A8 routes
    and the W8A8 comparator) on both MLP shapes."""
    a = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    (ng, kg), (nd, kd) = S.MLP_GATE_UP, S.MLP_DOWN
    blocks = mlp_layers(w, torch, S, COPIES)
    x_in = torch.from_numpy(S.activations(1, kg, seed=0)).cuda()
    x_hid = torch.from_numpy(S.activations(1, kd, seed=1)).cuda()
    xq_in, sx_in = w.prepare_activation(x_in)
    xq_hid, sx_hid = w.prepare_activation(x_hid)
    y_gu = [torch.empty((1, ng), dtype=torch.float32, device="cuda") for _ in range(2)]
    y_dn = torch.empty((1, nd), dtype=torch.float32, device="cuda")
    for c in range(COPIES):
        w.forward_multi(x_in, [blocks[c]["gate"], blocks[c]["up"]], outs=y_gu, x_q=xq_in, s_x=sx_in)
    for c in range(COPIES):
        w.forward(x_hid, blocks[c]["down"], out=y_dn, x_q=xq_hid, s_x=sx_hid)
    for c in range(COPIES):
        w.linear(xq_in, sx_in, blocks[c]["gate"], out=y_gu[0], algo=w.ALGO_GEMV)
        w.linear(xq_hid, sx_hid, blocks[c]["down"], out=y_dn, algo=w.ALGO_GEMV)
    torch.cuda.synchronize()
    for (n, k), L in ((S.MLP_GATE_UP, blocks[0]["gate"]), (S.MLP_DOWN, blocks[0]["down"])):
        xq, sx = w.prepare_activation(torch.from_numpy(S.activations(2048, k, seed=0)).cuda())
        y = torch.empty((2048, n), dtype=torch.float32, device="cuda")
        for algo in (w.ALGO_MFMA_I8, w.ALGO_MFMA_F16, w.ALGO_MFMA_RQ, w.ALGO_MFMA_I8_FOLD):
            w.linear(xq, sx, L, out=y, algo=algo)
        W8 = w.w8a8_quantize_weight(torch.from_numpy(S.weights(n, k, seed=0)).cuda())
        w.w8a8_linear(xq, sx, W8, out=y, algo=w.ALGO_MFMA_I8)
        del W8
    torch.cuda.synchronize()
    log("pmc pass done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-model", action="store_true")
    ap.add_argument("--no-quantize", action="store_true")
    ap.add_argument("--no-w8a8", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path (how the layer would shard is described with the design)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic as S
    import w4a8_codebook_gemm_amd as w

    torch.cuda.set_device(0)
    w.lib()
    shapes = [S.MLP_GATE_UP, S.MLP_DOWN]
    if args.pmc_pass:
        pmc_pass(w, torch, S, shapes)
        return

    d = decode(w, torch, S, args, shapes)
    torch.cuda.empty_cache()
    out = {
        "metric": METRIC, "value": round(d["value"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": d["warm"], "ms_per_step": round(d["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode M=1 of a 27B-class MLP block: rotate + int8-quantise + W4A8 "
                               "product, gate and up 17408x5120 in one fused launch "
                               "(w4a8_forward_multi), down 5120x17408 in a second (w4a8_forward); "
                               f"{COPIES} distinct weight copies of the block",
                   "tokens": 1, "weight_bytes_per_step": d["wb"]},
        "tokens_per_s": d["tokens_per_s"],
        "unfused_step_us": d["unfused_step_us"],
        "roofline": d["roofline"],
        "gemv": d["gemv"],
        "down": d["down"],
    }
    if not args.no_sweep:
        out["sweep"] = sweep(w, torch, S)
        torch.cuda.empty_cache()
    if not args.no_model:
        out["model"] = model(w, torch, S)
        torch.cuda.empty_cache()
    if not args.no_prefill:
        out["prefill"] = prefill(w, torch, S, shapes)
        torch.cuda.empty_cache()
    if not args.no_w8a8:
        out["w8a8"] = w8a8(w, torch, S, shapes, d["gemv"], d["unfused_step_us"], out.get("prefill"))
        torch.cuda.empty_cache()
    if not args.no_quantize:
        out["quantize"] = quantize_rate(w, torch, S, shapes)
        torch.cuda.empty_cache()
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(shapes)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
