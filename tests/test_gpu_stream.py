"""GPU parity of the T = 8 layer stream as the benchmark runs it: many independent 27B-like MLP
layers (H = 5120, I = 17408), each with its own seeded weights, signs and input, forwarded back to
back from one captured HIP graph on one shared workspace (the fused kernel's call epoch advances
and its operand buffers alternate between calls).  Every layer of every replay is compared with
the FP64 oracle; replays are also compared with an eager run bit for bit.

Bars as in test_gpu_parity: relative Frobenius error <= 2e-3 per layer, worst token row and worst
element within 1% of their row's scale.
"""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from bit_vector_lut_amd import synth

pytestmark = pytest.mark.gpu

MLP_TOL = 2e-3
LOCAL_TOL = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(name, y, ref):
    assert np.isfinite(y).all(), name
    err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    row = (np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)).max()
    elem = (np.abs(y - ref) / np.abs(ref).max(axis=1, keepdims=True)).max()
    assert err <= MLP_TOL and row <= LOCAL_TOL and elem <= LOCAL_TOL, (name, err, row, elem)
    return err, row, elem


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.fixture(scope="module")
def vq(torch_dev):
    from bit_vector_lut_amd import vqmlp

    vqmlp.lib()
    return vqmlp


def _layer_job(i, n_layers):
    from bit_vector_lut_amd import vqmlp

    L = synth.stream_layer(i, n_layers)
    return L, [vqmlp.pack(*m.as_u16()) for m in (L.gate, L.up, L.down)]


def _build_stream(vq, oracle_mod, n_layers, device="cuda"):
    """Layers in order: drawn and packed on worker threads (a few at a time), the oracle's output
    computed on the host, the packed weights uploaded; host copies are dropped as we go."""
    mlps, xs, refs = [], [], []
    with ThreadPoolExecutor(max_workers=4) as ex:
        pending = [ex.submit(_layer_job, i, n_layers) for i in range(min(4, n_layers))]
        for i in range(n_layers):
            L, packs = pending.pop(0).result()
            if i + len(pending) + 1 < n_layers:
                pending.append(ex.submit(_layer_job, i + len(pending) + 1, n_layers))
            refs.append(oracle_mod.mlp_forward(L))
            dev = [vq.to_device(p, device) for p in packs]
            mlps.append(vq.MLP(L.H, L.I, *dev, vq.to_device(L.s, device),
                               vq.to_device(L.sign_h, device), vq.to_device(L.sign_i, device),
                               L.had_block_h, L.had_block_i, t_max=8))
            xs.append(vq.to_device(L.x, device))
            del L, packs
            if (i + 1) % 16 == 0:
                _say("stream: %d/%d layers ready" % (i + 1, n_layers))
    return mlps, xs, refs


def test_stream_64_layers_graph_replays_match_oracle(vq, oracle_mod, torch_dev):
    torch = torch_dev
    n_layers = 64
    _say("stream: building %d layers" % n_layers)
    mlps, xs, refs = _build_stream(vq, oracle_mod, n_layers)
    ws = mlps[0].workspace(8)
    ys = [torch.empty_like(x) for x in xs]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for m, x, y in zip(mlps, xs, ys):
            m.forward(x, y, ws, stream=st)
    st.synchronize()
    eager = [y.clone() for y in ys]
    assert vq.workspace_errors(ws, stream=st) == 0
    worst = (0.0, 0.0, 0.0)
    for i, (y, ref) in enumerate(zip(eager, refs)):
        got = y.cpu().numpy().view(np.float16).astype(np.float64)
        worst = tuple(max(a, b) for a, b in zip(worst, _check("eager layer %d" % i, got, ref)))
    _say("stream eager: worst rel_fro=%.3e worst_row=%.3e worst_elem=%.3e" % worst)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for m, x, y in zip(mlps, xs, ys):
            m.forward(x, y, ws, stream=st)
    for rep in range(3):
        for y in ys:
            y.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g.replay()
        st.synchronize()
        assert vq.workspace_errors(ws, stream=st) == 0, "replay %d: a wait ran out" % rep
        for i, (y, ref) in enumerate(zip(ys, refs)):
            assert torch.equal(y, eager[i]), "replay %d layer %d differs from eager" % (rep, i)
            if rep == 0:
                got = y.cpu().numpy().view(np.float16).astype(np.float64)
                _check("replay %d layer %d" % (rep, i), got, ref)
        _say("stream replay %d: all %d layers bitwise equal to eager" % (rep, n_layers))
        # eager work on the same workspace between replays (the epoch keeps counting)
        with torch.cuda.stream(st):
            mlps[rep].forward(xs[rep], ys[rep], ws, stream=st)
        st.synchronize()
        assert torch.equal(ys[rep], eager[rep])


@pytest.mark.parametrize("H,I,T", [(512, 1024, 8), (256, 704, 3), (1024, 2048, 5)])
def test_fused_graph_of_distinct_layers(vq, oracle_mod, torch_dev, H, I, T):
    """Small layers of one shape in one graph on one workspace, replayed several times with eager
    forwards and synchronisations between replays: every replay equals the eager results bit for
    bit and the oracle within the bars."""
    torch = torch_dev
    layers = [synth.mlp_layer(H, I, T, seed=100 + i, outliers=True) for i in range(5)]
    mlps = [vq.MLP.from_layer(L, t_max=8) for L in layers]
    xs = [vq.to_device(L.x) for L in layers]
    refs = [oracle_mod.mlp_forward(L) for L in layers]
    ws = mlps[0].workspace(8)
    ys = [torch.empty_like(x) for x in xs]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for m, x, y in zip(mlps, xs, ys):
            m.forward(x, y, ws, stream=st)
    st.synchronize()
    eager = [y.clone() for y in ys]
    for i, (y, ref) in enumerate(zip(eager, refs)):
        _check("eager %d" % i, y.cpu().numpy().view(np.float16).astype(np.float64), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for m, x, y in zip(mlps, xs, ys):
            m.forward(x, y, ws, stream=st)
    for rep in range(4):
        for y in ys:
            y.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g.replay()
        st.synchronize()
        for i, y in enumerate(ys):
            assert torch.equal(y, eager[i]), "replay %d layer %d" % (rep, i)
        with torch.cuda.stream(st):
            mlps[-1].forward(xs[-1], ys[-1], ws, stream=st)
        st.synchronize()
    assert vq.workspace_errors(ws, stream=st) == 0
