"""Benchmark of the VQ3 quantized-MLP forward on one MI355X.

A step is one pass of the T=8 hot path over the 64-layer stream: 64 independent 27B-like MLP
layers (H=5120, I=17408), each with its own seeded codes, codebooks, scales, signs and input,
run back to back from one captured HIP graph.  The weights (6.5 GB) exceed every on-die cache,
so the stream is HBM-bound.  The metric is the effective weight bandwidth: algorithmic weight
bytes (codes at exactly 3 bits per weight + codebooks + row scales) per second.

Beside it: the T=512 prefill MLP (TFLOP/s against the FP16 matrix-core peak), the roofline of
the dominant kernel, and the FP64 CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--layers 64] [--no-cpu] [--no-t512]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I = 5120, 17408
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 matrix cores, published


def weight_bytes(H, I):
    """Algorithmic bytes of one layer: 3-bit codes + 64x2 FP16 codebooks per 8 rows + FP16 row
    scales, for gate (I x H), up (I x H) and down (H x I)."""
    per = lambda N, K: N * K * 3 // 8 + (N // 8) * 64 * 2 * 2 + N * 2
    return 2 * per(I, H) + per(H, I)


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_fused_t8_27b_traffic.txt")
KERNEL_SOURCES = ["fused.hip", "device.h", "internal.h"]


def kernel_source_hash():
    """SHA-256 of the sources the fused kernel is compiled from and of its compiler flags."""
    import hashlib

    from bit_vector_lut_amd import build as hipbuild

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_vector_lut_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(hipbuild.HIP_FLAGS + hipbuild.SOURCE_FLAGS.get("fused.hip", [])).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the fused kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads for a copy of known size),
    or None when that summary was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def probe(device, t512=False):
    """Counter run (under rocprofv3 --pmc): two kernels of known size to scale the byte counters
    (a 256 MiB device copy, and one streaming read of the same 256 MiB with the library's read
    kernel), then four fused T=8 forwards on four distinct seeded layers; with t512, two T=512
    forwards of the prefill layer instead of the T=8 ones."""
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    vqmlp.stream_read(src, sink)
    torch.cuda.synchronize()
    del src, dst
    if t512:
        L5, _, _ = synth.prefill512()
        m5 = vqmlp.MLP.from_layer(L5, device=device, t_max=512)
        x5 = vqmlp.to_device(L5.x, device)
        ws5 = m5.workspace(512)
        for _ in range(2):
            m5.forward(x5, torch.empty_like(x5), ws5)
        torch.cuda.synchronize()
        log("probe done: copy and read of %d bytes, 2 T=512 forwards" % n)
        return
    layers = build_stream(4, device)
    ws = layers[0][0].workspace(8)
    for m, x in layers:
        m.forward(x, torch.empty_like(x), ws)
    torch.cuda.synchronize()
    log("probe done: copy and read of %d bytes, %d forwards" % (n, len(layers)))


def build_stream(n_layers, device, t_max=64):
    """Generate, pack and upload the layer stream (host copies dropped as we go)."""
    import torch  # noqa: F401
    from concurrent.futures import ThreadPoolExecutor

    from bit_vector_lut_amd import synth, vqmlp

    def job(i):
        L = synth.stream_layer(i)
        packs = [vqmlp.pack(*m.as_u16()) for m in (L.gate, L.up, L.down)]
        return L, packs

    layers = []
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for i, (L, packs) in enumerate(ex.map(job, range(n_layers))):
            dev = [vqmlp.to_device(p, device) for p in packs]
            mlp = vqmlp.MLP(H, I, *dev, vqmlp.to_device(L.s, device),
                            vqmlp.to_device(L.sign_h, device), vqmlp.to_device(L.sign_i, device),
                            L.had_block_h, L.had_block_i, t_max=t_max)
            layers.append((mlp, vqmlp.to_device(L.x, device)))
            if i == 0 or (i + 1) % 16 == 0:
                log("layer %d/%d ready (%.1f s)" % (i + 1, n_layers, time.time() - t0))
    return layers


def host_cpu():
    """Model name of the host CPU and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, usable


def timed_events(stream, fn, reps):
    """Average ms of fn() over reps calls, HIP events on `stream` around the calls."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def capture(stream, fn):
    """A HIP graph of fn() captured on `stream` (after one eager run)."""
    import torch

    with torch.cuda.stream(stream):
        fn()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def extra_lines(device, stream, layers):
    """The single-layer workloads: the tiny layer (H 256, I 704, T 1: launch-bound, microseconds),
    one 27B-like layer at T = 8 with its weights hot in the on-die cache and cold (a 1 GiB write
    between timed forwards evicts them), the 27B-like layers at T = 64 (the fixed prefill chunk;
    a graph over the stream's layers so the weights come from HBM), and the streaming-read rate
    of this GPU's HBM with the library's own read kernel."""
    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    out = {}
    # tiny layer, T = 1
    L1 = synth.tiny_layer()
    m1 = vqmlp.MLP.from_layer(L1, device=device, t_max=8)
    x1 = vqmlp.to_device(L1.x, device)
    y1 = torch.empty_like(x1)
    w1 = m1.workspace(8)
    with torch.cuda.stream(stream):
        for _ in range(20):
            m1.forward(x1, y1, w1, stream=stream)
        eager_us = timed_events(stream, lambda: m1.forward(x1, y1, w1, stream=stream), 200) * 1e3
    g1 = capture(stream, lambda: [m1.forward(x1, y1, w1, stream=stream) for _ in range(100)])
    with torch.cuda.stream(stream):
        g1.replay()
        graph_us = timed_events(stream, g1.replay, 20) * 1e3 / 100
    out["tiny_t1"] = {"workload": "tiny MLP layer H=256 I=704 T=1 (259,328 weight bytes)",
                      "us_eager": round(eager_us, 2), "us_graph": round(graph_us, 2)}
    log("tiny layer T=1: %.2f us per forward (back-to-back launches), %.2f us (graph)" %
        (eager_us, graph_us))
    del g1

    # one 27B-like layer at T = 8, hot and cold
    L2 = synth.layer27b_t8()
    m2 = vqmlp.MLP.from_layer(L2, device=device, t_max=8)
    x2 = vqmlp.to_device(L2.x, device)
    y2 = torch.empty_like(x2)
    w2 = m2.workspace(8)
    del L2
    with torch.cuda.stream(stream):
        for _ in range(5):
            m2.forward(x2, y2, w2, stream=stream)
        hot_us = timed_events(stream, lambda: m2.forward(x2, y2, w2, stream=stream), 50) * 1e3
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device=device)
        cold = []
        for i in range(20):
            scrub.fill_(i & 255)
            cold.append(timed_events(stream, lambda: m2.forward(x2, y2, w2, stream=stream), 1))
        del scrub
    cold_us = float(np.median(cold)) * 1e3
    wb = weight_bytes(H, I)
    out["layer27b_t8"] = {
        "workload": "one 27B-like layer H=5120 I=17408 T=8, 1% outlier channels x20, seed 0",
        "us_hot": round(hot_us, 2), "gbps_hot": round(wb / hot_us / 1e3, 1),
        "us_cold": round(cold_us, 2), "gbps_cold": round(wb / cold_us / 1e3, 1),
        "frac_hbm_cold": round(wb / cold_us / 1e3 / HBM_PEAK_GBS, 4),
        "cold": "median of 20 forwards, each after an untimed 1 GiB write"}
    log("27B-like layer T=8: hot %.1f us (%.0f GB/s), cold %.1f us (%.0f GB/s)" %
        (hot_us, wb / hot_us / 1e3, cold_us, wb / cold_us / 1e3))
    del m2, x2, y2, w2

    # T = 64 over the stream's layers (weights from HBM), one graph of all forwards
    rng = np.random.default_rng(64)
    x64 = [vqmlp.to_device(synth.activations(rng, 64, H, False), device) for _ in layers]
    y64 = [torch.empty_like(x) for x in x64]
    w64 = layers[0][0].workspace(64)
    g64 = capture(stream, lambda: [m.forward(x, y, w64, stream=stream)
                                   for (m, _), x, y in zip(layers, x64, y64)])
    with torch.cuda.stream(stream):
        g64.replay()
        us64 = timed_events(stream, g64.replay, 5) * 1e3 / len(layers)
    flops64 = 2.0 * 64 * 3 * H * I
    out["layer27b_t64"] = {
        "workload": "27B-like layers at T=64 (fixed prefill chunk), inputs N(0,1), one graph over "
                    "the %d stream layers" % len(layers),
        "us": round(us64, 2), "gbps": round(wb / us64 / 1e3, 1),
        "frac_hbm": round(wb / us64 / 1e3 / HBM_PEAK_GBS, 4),
        "tflops": round(flops64 / us64 / 1e6, 1),
        "frac_mfma": round(flops64 / us64 / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)}
    log("27B-like layer T=64: %.1f us, %.0f GB/s, %.1f TFLOP/s" % (us64, wb / us64 / 1e3,
                                                                  flops64 / us64 / 1e6))
    del g64, x64, y64, w64

    # streaming read over 4 GiB
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=device).fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    with torch.cuda.stream(stream):
        vqmlp.stream_read(buf, sink, stream)
        ms = timed_events(stream, lambda: vqmlp.stream_read(buf, sink, stream), 10)
    rd = buf.numel() / (ms * 1e-3) / 1e9
    out["achievable_read"] = {"bytes": buf.numel(), "us": round(ms * 1e3, 1), "gbps": round(rd, 1),
                              "frac_hbm": round(rd / HBM_PEAK_GBS, 4),
                              "kernel": "k_stream_read (16-byte loads, contiguous share per "
                                        "workgroup, 8 workgroups per CU)"}
    log("streaming read of 4 GiB: %.1f GB/s" % rd)
    del buf
    return out


def lut_weight_bytes(bits, N, K, r):
    """Bytes one scalar-LUT projection reads from its weights: codes (bits per weight), tables
    (2^bits binary16 per 8 rows), row scales (binary16), U [N][r] and V [r][K] (binary16)."""
    return N * K * bits // 8 + (N // 8) * (1 << bits) * 2 + N * 2 + r * (N + K) * 2


def t8_mixers(device, stream, n_proj=16):
    """The token-mixer projections at T = 8 (5120 x 5120, rank 64, 1024-wide rotation): one HIP
    graph of n_proj distinct seeded projections per code width (more bytes than the on-die cache
    holds), timed over replays; effective weight GB/s against the HBM peak."""
    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    out = []
    for bits in (2, 4):
        projs = [vqmlp.LUTProjection.from_proj(
            synth.lut_projection(np.random.default_rng(9000 + 100 * bits + i), bits, 5120, 5120, 64, 1024),
            device) for i in range(n_proj)]
        x = vqmlp.to_device(synth.activations(np.random.default_rng(bits), 8, 5120, True), device)
        ys = [torch.empty((8, 5120), dtype=x.dtype, device=device) for _ in projs]
        ws = projs[0].workspace(8)
        with torch.cuda.stream(stream):
            for m, y in zip(projs, ys):
                m.forward(x, y, ws, stream=stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for m, y in zip(projs, ys):
                m.forward(x, y, ws, stream=stream)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            with torch.cuda.stream(stream):
                g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n_proj)
        wb = lut_weight_bytes(bits, 5120, 5120, 64)
        gbs = wb / (us * 1e-6) / 1e9
        log("T=8 %d-bit mixer 5120x5120 r=64: %.2f us per forward, %.1f GB/s of weights" % (bits, us, gbs))
        out.append({"bits": bits, "N": 5120, "K": 5120, "rank": 64, "T": 8, "us": round(us, 2),
                    "weight_bytes": wb, "gbps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        del g, projs, ys
    return out


def t8_vq2(device, stream, n_proj=16):
    """The 2x16 vector-LUT projection at T = 8 (5120 x 5120 and the 17408 x 5120 gate / up shape):
    one HIP graph of n_proj distinct seeded matrices per shape, timed over replays; weight GB/s
    (codes, centroids, scales) against the HBM peak."""
    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    out = []
    for N, K in ((5120, 5120), (17408, 5120)):
        projs = [vqmlp.VQ2Projection.from_matrix(
            synth.vq2_matrix(np.random.default_rng(7000 + i), N, K), device) for i in range(n_proj)]
        x = vqmlp.to_device(synth.activations(np.random.default_rng(N), 8, K, True), device)
        ys = [torch.empty((8, N), dtype=x.dtype, device=device) for _ in projs]
        with torch.cuda.stream(stream):
            for m, y in zip(projs, ys):
                m.forward(x, y, stream=stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for m, y in zip(projs, ys):
                m.forward(x, y, stream=stream)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            with torch.cuda.stream(stream):
                g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n_proj)
        wb = N * K // 4 + (N // 8) * 16 * 4 + N * 2
        gbs = wb / (us * 1e-6) / 1e9
        log("T=8 2x16 projection %dx%d: %.2f us per forward, %.1f GB/s of weights" % (N, K, us, gbs))
        out.append({"N": N, "K": K, "T": 8, "us": round(us, 2), "weight_bytes": wb,
                    "gbps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        del g, projs, ys
    return out


def vq2_weight_bytes(H, I):
    """Algorithmic bytes of one 2x16 layer: 4-bit codes per pair of rows (2 bits per weight),
    16 two-component binary16 centroids per 8 rows, binary16 row scales; gate, up and down."""
    per = lambda N, K: N * K // 4 + (N // 8) * 16 * 4 + N * 2
    return 2 * per(I, H) + per(H, I)


def vq2_mlp_lines(device, stream, n_layers=8):
    """The 2x16 MLP (previous packages' format) at the 27B-like shape: a graph of n_layers
    distinct seeded layers (more bytes than the on-die cache), at T = 8 and at T = 64."""
    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    mlps, xs8, xs64 = [], [], []
    for i in range(n_layers):
        L = synth.vq2_mlp_layer(H, I, 8, seed=8000 + i, outliers=True)
        mlps.append(vqmlp.MLP.from_vq2_layer(L, device=device, t_max=64))
        xs8.append(vqmlp.to_device(L.x, device))
        xs64.append(vqmlp.to_device(synth.activations(np.random.default_rng(8100 + i), 64, H, False),
                                    device))
        del L
    wb = vq2_weight_bytes(H, I)
    out = {"workload": "27B-like MLP in the 2x16 format (H=5120, I=17408), graph of %d layers" % n_layers,
           "weight_bytes_per_layer": wb}
    for T, xs in ((8, xs8), (64, xs64)):
        ys = [torch.empty_like(x) for x in xs]
        ws = mlps[0].workspace(T)
        g = capture(stream, lambda: [m.forward(x, y, ws, stream=stream) for m, x, y in zip(mlps, xs, ys)])
        with torch.cuda.stream(stream):
            g.replay()
            us = timed_events(stream, g.replay, 10) * 1e3 / n_layers
        fl = 2.0 * T * 3 * H * I
        out["t%d" % T] = {"us": round(us, 2), "gbps": round(wb / us / 1e3, 1),
                          "frac_hbm": round(wb / us / 1e3 / HBM_PEAK_GBS, 4),
                          "tflops": round(fl / us / 1e6, 1)}
        log("2x16 MLP T=%d: %.1f us per layer, %.0f GB/s of weights, %.1f TFLOP/s" % (
            T, us, wb / us / 1e3, fl / us / 1e6))
        del g, ys, ws
    return out


def t8_lm_head(device, stream):
    """The four-bit LUT output head (248,320 x 5120) with in-model argmax at T = 8: one seeded
    head (636 MB of codes, more than the on-die cache), timed over back-to-back calls with
    events on the stream they run on; effective weight GB/s against the HBM peak."""
    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    N, K, T = 248320, 5120, 8
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    lut = (rng.standard_normal((N // 8, 16)) * 0.02).astype(np.float16)
    sc = rng.uniform(0.5, 1.5, N).astype(np.float16)
    packed = vqmlp.to_device(vqmlp.lut_pack(4, codes, lut, sc), device)
    del codes
    head = vqmlp.LUTProjection(4, N, K, packed, None, None, None, None, 0)
    x = vqmlp.to_device(synth.activations(rng, T, K, True), device)
    ws = head.workspace(T)
    with torch.cuda.stream(stream):
        for _ in range(2):
            head.argmax(x, ws, stream=stream)
    stream.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            head.argmax(x, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    wb = lut_weight_bytes(4, N, K, 0)
    gbs = wb / (us * 1e-6) / 1e9
    log("T=8 LM head 4-bit %dx%d + argmax: %.1f us, %.1f GB/s of weights" % (N, K, us, gbs))
    return {"bits": 4, "N": N, "K": K, "T": T, "us": round(us, 1), "weight_bytes": wb,
            "gbps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-t512", action="store_true")
    ap.add_argument("--no-mixers8", action="store_true")
    ap.add_argument("--no-vq2", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the tiny, single-layer, T=64 and streaming-read lines")
    ap.add_argument("--probe", action="store_true",
                    help="counter run only: known-size copy and read, 4 T=8 forwards, no timing")
    ap.add_argument("--probe512", action="store_true",
                    help="counter run only: known-size copy and read, 2 T=512 forwards")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d "
              "requested); run with --gpus 1" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    device = "cuda:0"
    torch.cuda.set_device(0)
    vqmlp.lib()
    if args.probe or args.probe512:
        probe(device, t512=args.probe512)
        return

    # ---------------------------------------------------------------- T = 8, 64-layer stream
    layers = build_stream(args.layers, device)
    ws = layers[0][0].workspace(8)
    ys = [torch.empty_like(x) for _, x in layers]
    stream = torch.cuda.Stream()
    log("capturing the %d-layer graph" % len(layers))
    graph = capture(stream, lambda: [m.forward(x, y, ws, stream=stream)
                                     for (m, x), y in zip(layers, ys)])
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    stream.synchronize()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ms_step = timed_events(stream, graph.replay, args.steps)
    torch.cuda.synchronize()
    bytes_step = weight_bytes(H, I) * len(layers)
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    log("T=8 stream: %.3f ms/step, %.1f GB/s" % (ms_step, gbs))
    err_bits = vqmlp.workspace_errors(ws, stream=stream)
    if err_bits:
        log("FAILED: a bounded wait of the fused kernel ran out (error bits %#x)" % err_bits)
        sys.exit(3)

    # the replayed outputs of the first and last layers against the oracle
    from oracle import oracle as O

    parity = {"tol_rel_fro": 2e-3, "layers": [], "rel_fro": [], "worst_row": []}
    oracle_s = None
    for li in sorted({0, len(layers) - 1}):
        L = synth.stream_layer(li)
        t0 = time.time()
        ref = O.mlp_forward(L)
        if li == 0:
            oracle_s = time.time() - t0
        got = ys[li].cpu().numpy().view(np.float16).astype(np.float64)
        err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        row = float((np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)).max())
        parity["layers"].append(li)
        parity["rel_fro"].append(round(err, 6))
        parity["worst_row"].append(round(row, 6))
        log("layer %d of the replayed stream against the oracle: rel_fro %.3e, worst row %.3e" %
            (li, err, row))
        del L
    parity["ok"] = all(e <= 2e-3 for e in parity["rel_fro"])
    if not parity["ok"]:
        log("FAILED: stream output outside the tolerance")
        print(json.dumps({"parity": parity}), flush=True)
        sys.exit(4)

    # dominant kernel: the T = 8 forward is one launch of the fused kernel; its average launch
    # duration is timed with events on the stream it runs on, over back-to-back launches that
    # cycle through the layers so that every launch reads weights that are not cache-resident
    n_fw = len(layers)

    def all_layers():
        for i in range(n_fw):
            layers[i][0].forward(layers[i][1], ys[i], ws, stream=stream)

    with torch.cuda.stream(stream):
        all_layers()  # warm
        fw_ms = timed_events(stream, all_layers, 3) / n_fw
    fw_gbs = weight_bytes(H, I) / (fw_ms * 1e-3) / 1e9
    log("fused forward launch (events, %d back-to-back): %.1f us, %.1f GB/s" % (3 * n_fw,
                                                                              fw_ms * 1e3, fw_gbs))
    traffic = measured_traffic()

    result = {
        "metric": "VQ3 MLP effective weight GB/s at T=8 + TFLOP/s at T=512, % of roofline",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 operands / f32 accumulate (3-bit VQ weights)",
        "data": "synthetic",
        "config": {"workload": "64 independent 27B-like VQ3 MLP layers streamed at T=8 "
                               "(H=5120, I=17408, one HIP graph, 6.50 GB of weights)",
                   "layers": len(layers), "T": 8, "H": H, "I": I,
                   "weight_bytes_per_layer": weight_bytes(H, I)},
        "roofline": {"bound": "hbm", "kernel": "k_fused<5> (whole T=8 forward of one layer, one launch)",
                     "achieved": round(fw_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fw_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": weight_bytes(H, I),
                     "us_per_launch": round(fw_ms * 1e3, 2)},
        "parity": parity,
        "fused_error_bits": err_bits,
    }
    del graph

    if not args.no_extra:
        result.update(extra_lines(device, stream, layers))

    # ---------------------------------------------------------------- T = 8 token mixers
    if not args.no_mixers8:
        result["t8_token_mixers"] = t8_mixers(device, stream)
    if not args.no_vq2:
        result["t8_vq2x16"] = t8_vq2(device, stream)
        result["t8_lm_head_argmax"] = t8_lm_head(device, stream)
        result["vq2x16_mlp"] = vq2_mlp_lines(device, stream)

    # ---------------------------------------------------------------- T = 512 prefill MLP
    if not args.no_t512:
        del ys
        L5, p2, p4 = synth.prefill512()
        m5 = vqmlp.MLP.from_layer(L5, device=device, t_max=512)
        mixers = [vqmlp.LUTProjection.from_proj(p, device) for p in (p2, p4)]
        x5 = vqmlp.to_device(L5.x, device)
        y5 = torch.empty_like(x5)
        ws5 = m5.workspace(512)
        ym = [torch.empty((512, p.N), dtype=x5.dtype, device=device) for p in (p2, p4)]
        wsm = [mx.workspace(512) for mx in mixers]
        reps = 10

        def timed(fn):
            """(eager ms, graph ms) per call: back-to-back calls, and replays of a graph of one."""
            with torch.cuda.stream(stream):
                for _ in range(3):
                    fn()
                eager = timed_events(stream, fn, reps)
            g = capture(stream, fn)
            with torch.cuda.stream(stream):
                g.replay()
                graphed = timed_events(stream, g.replay, reps)
            return eager, graphed

        ms5e, ms5 = timed(lambda: m5.forward(x5, y5, ws5, stream=stream))
        ms_mix = [timed(lambda mx=mx, y=y, w=w: mx.forward(x5, y, w, stream=stream))
                  for mx, y, w in zip(mixers, ym, wsm)]
        flops = 2.0 * 512 * 3 * H * I
        tf = flops / (ms5 * 1e-3) / 1e12
        log("T=512 MLP: %.1f us (graph), %.1f us (back-to-back), %.1f TFLOP/s" % (
            ms5 * 1e3, ms5e * 1e3, tf))
        result["t512"] = {"workload": "27B-like VQ3 MLP prefill, T=512", "us": round(ms5 * 1e3, 1),
                          "us_eager": round(ms5e * 1e3, 1),
                          "tflops": round(tf, 1), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                          "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "token_mixers": []}
        for p, (mse, ms) in zip((p2, p4), ms_mix):
            fl = 2.0 * 512 * (p.N * p.K + p.rank * (p.N + p.K))
            tfm = fl / (ms * 1e-3) / 1e12
            log("T=512 %d-bit mixer %dx%d r=%d: %.1f us (graph), %.1f TFLOP/s" % (
                p.bits, p.N, p.K, p.rank, ms * 1e3, tfm))
            result["t512"]["token_mixers"].append(
                {"bits": p.bits, "N": p.N, "K": p.K, "rank": p.rank, "us": round(ms * 1e3, 1),
                 "us_eager": round(mse * 1e3, 1),
                 "tflops": round(tfm, 1), "frac": round(tfm / MFMA_F16_PEAK_TFLOPS, 4)})

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu:
        model, usable = host_cpu()
        all_threads = O.num_threads()
        L0 = synth.stream_layer(0)
        O.set_num_threads(1)
        t0 = time.time()
        O.mlp_forward(L0)
        one_s = time.time() - t0
        O.set_num_threads(all_threads)
        wb = weight_bytes(H, I)
        result["cpu_baseline"] = {
            "value": round(wb / oracle_s / 1e9, 5), "unit": "GB/s", "cores": all_threads,
            "kind": "oracle",
            "sample": "layer 0 of the 64-layer stream, all 8 tokens: one full FP64 forward "
                      "(%.2f s on %d threads; %.2f s on 1 thread)" % (oracle_s, all_threads, one_s),
            "value_1_thread": round(wb / one_s / 1e9, 5),
            "host_cpu": model, "usable_cores": usable}
        log("oracle: %.2f s for one layer on %d threads, %.2f s on 1 thread (%s, %d usable cores)"
            % (oracle_s, all_threads, one_s, model, usable))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
