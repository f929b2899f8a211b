"""GPU: a NaN-poisoned workspace gives the same outputs, bit for bit, as a zeroed one.

Every byte of the workspace is set to 0xFF (a NaN as binary16 and as FP32, and a tag no call ever
uses) except the MLP's 64-byte control block, which the interface asks the caller to zero once.
Two calls in a row on the poisoned workspace must then reproduce the outputs of a call on a
zeroed workspace exactly: no kernel may read a workspace byte that the same call has not written
first (K-split planes, rotated operands, rank-r partial sums, the argmax candidates), and the
fused kernel's tagged hand-off words must not take a poisoned word for this call's data.
Shapes reach every kernel family: the fused T <= 8 kernel, the tiled and register-decode products
with their K splits (gate/up combine and down reduction), the 2x16 paths, the scalar-LUT
projections at T <= 8 and from T = 33, and the argmax head.
"""
import sys

import numpy as np
import pytest

from bit_vector_lut_amd import synth

pytestmark = pytest.mark.gpu

CTL_BYTES = 64  # the control block the caller zero-fills once (MLP plans)


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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _poisoned(torch, nbytes, ctl_bytes):
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    if ctl_bytes:
        ws[:ctl_bytes] = 0
    return ws


def _same(torch, a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _check_mlp(vq, torch, mlp, x, path, name):
    T = x.shape[0]
    nbytes = mlp.workspace_bytes(T)
    ref = mlp.forward(x, workspace=mlp.workspace(T), path=path)
    ws = _poisoned(torch, nbytes, CTL_BYTES)
    for call in range(2):
        y = torch.full_like(x, 0x7E00)  # binary16 NaN: every output must be written
        mlp.forward(x, y, ws, path=path)
        torch.cuda.synchronize()
        _say("%s call %d: %d workspace bytes poisoned" % (name, call, nbytes - CTL_BYTES))
        assert _same(torch, y, ref), "%s: call %d on a poisoned workspace differs" % (name, call)
    assert vq.workspace_errors(ws) == 0, "%s: a bounded wait ran out" % name


@pytest.mark.parametrize("H,I,T,path", [
    (1024, 2048, 1, 1), (1024, 2048, 8, 1), (256, 704, 5, 1),      # fused T <= 8 kernel
    (1024, 2048, 8, 2), (1024, 2048, 16, 2),                        # tiled products
    (1024, 2048, 48, 2), (1024, 4352, 300, 2), (256, 704, 130, 2),  # register-decode, K splits
])
def test_poisoned_workspace_mlp(vq, torch_dev, H, I, T, path):
    torch = torch_dev
    layer = synth.mlp_layer(H, I, T, seed=H + I + T, outliers=True)
    mlp = vq.MLP.from_layer(layer, t_max=max(T, 8))
    x = vq.to_device(layer.x)
    _check_mlp(vq, torch, mlp, x, path, "mlp H=%d I=%d T=%d path %d" % (H, I, T, path))


@pytest.mark.parametrize("T", [8, 64, 512])
def test_poisoned_workspace_mlp_27b(vq, torch_dev, T):
    """The 27B-like shape: the fused kernel's four down slices (T = 8), the gate/up K split with
    its combine pass and the ten-way down split (T = 64), the leftover rows' K split beside the
    main tiles (T = 512)."""
    torch = torch_dev
    layer = synth.mlp_layer(5120, 17408, T, seed=1000 + T, outliers=T == 8)
    mlp = vq.MLP.from_layer(layer, t_max=T)
    x = vq.to_device(layer.x)
    del layer
    _check_mlp(vq, torch, mlp, x, 0, "mlp 27B-like T=%d" % T)


@pytest.mark.parametrize("H,I,T,path", [
    (1024, 2048, 8, 1),     # 2x16 projection kernel: gate/up planes, down slices
    (1024, 2048, 16, 2),    # tiled kernels with the 2x16 decoder
    (1024, 2048, 64, 2),    # register-decode kernels with the 2x16 decoder
])
def test_poisoned_workspace_vq2_mlp(vq, torch_dev, H, I, T, path):
    torch = torch_dev
    layer = synth.vq2_mlp_layer(H, I, T, seed=7 + T)
    mlp = vq.MLP.from_vq2_layer(layer, t_max=max(T, 8))
    x = vq.to_device(layer.x)
    _check_mlp(vq, torch, mlp, x, path, "2x16 mlp H=%d I=%d T=%d path %d" % (H, I, T, path))


@pytest.mark.parametrize("bits,N,K,T,rank", [
    (2, 1024, 2048, 8, 64), (4, 1024, 2048, 3, 64),   # T <= 8: pre-pass planes + product
    (2, 1024, 2048, 48, 64), (4, 1024, 2048, 300, 64),  # from T = 33: z = V x~ split, K-split planes
    (4, 512, 1024, 16, 0),                            # tiled product, no rank term
])
def test_poisoned_workspace_lut(vq, torch_dev, bits, N, K, T, rank):
    torch = torch_dev
    rng = np.random.default_rng(100 * bits + T)
    p = synth.lut_projection(rng, bits, N, K, rank, 1024)
    proj = vq.LUTProjection.from_proj(p)
    x = vq.to_device(rng.standard_normal((T, K)).astype(np.float16))
    ref = proj.forward(x, workspace=proj.workspace(T))
    nbytes = proj.workspace_bytes(T)
    ws = _poisoned(torch, nbytes, 0)
    for call in range(2):
        y = torch.full((T, N), 0x7E00, dtype=torch.int16, device="cuda").view(x.dtype)
        proj.forward(x, y, ws)
        torch.cuda.synchronize()
        _say("lut%d N=%d K=%d T=%d r=%d call %d" % (bits, N, K, T, rank, call))
        assert _same(torch, y, ref), "lut%d T=%d: call %d on a poisoned workspace differs" % (
            bits, T, call)


def test_poisoned_workspace_argmax(vq, torch_dev):
    torch = torch_dev
    rng = np.random.default_rng(77)
    p = synth.lut_projection(rng, 4, 4096, 1024, 0, 0)
    proj = vq.LUTProjection.from_proj(p)
    x = vq.to_device(rng.standard_normal((8, 1024)).astype(np.float16))
    ref_i, ref_v = proj.argmax(x, workspace=proj.workspace(8))
    ws = _poisoned(torch, proj.workspace_bytes(8), 0)
    for call in range(2):
        idx, val = proj.argmax(x, workspace=ws)
        torch.cuda.synchronize()
        _say("argmax head call %d: %s" % (call, idx.cpu().tolist()))
        assert torch.equal(idx, ref_i) and torch.equal(val.view(torch.int32), ref_v.view(torch.int32))
