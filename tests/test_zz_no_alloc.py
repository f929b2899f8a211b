"""GPU test of vqmlp_forward_noalloc (the forward whose workspace is the library's fixed per-GPU
scratch array): through the C ABI, its outputs equal vqmlp_forward's (same kernels) bit for bit,
on two calls in a row with the second one smaller, on the fused (T <= 8) and the tiled path;
a forward whose workspace would not fit is refused without a launch."""
import sys

import numpy as np
import pytest

from bit_vector_lut_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


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


def _pair(vq, torch, mlp, x):
    """(vqmlp_forward with a fresh zeroed workspace, vqmlp_forward_noalloc) on the same x."""
    y_ref = mlp.forward(x, workspace=mlp.workspace(x.shape[0]))
    y = torch.full_like(x, 0x7E00)  # NaN pattern: every output must be written
    mlp.forward_noalloc(x, y)
    torch.cuda.synchronize()
    return y_ref, y


def test_noalloc_matches_forward_27b(vq, oracle_mod, torch_dev):
    torch = torch_dev
    L = synth.layer27b_t8()
    mlp = vq.MLP.from_layer(L, t_max=512)
    _say("no-alloc 27B-like T=8: workspace %d bytes" % mlp.workspace_bytes(8))
    x = vq.to_device(L.x)
    y_ref, y = _pair(vq, torch, mlp, x)
    assert torch.equal(y, y_ref)
    got = y.cpu().numpy().view(np.float16).astype(np.float64)
    ref = oracle_mod.mlp_forward(L)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 2e-3
    # second call, smaller input (3 tokens), same scratch array
    x3 = x[:3].clone()
    _say("no-alloc 27B-like T=3")
    y_ref3, y3 = _pair(vq, torch, mlp, x3)
    assert torch.equal(y3, y_ref3)
    assert torch.equal(y3, y[:3])  # tokens are independent: the same bits as in the T=8 call
    # a forward whose workspace exceeds the array is refused, nothing launched
    _say("no-alloc 27B-like T=512: workspace %d bytes" % mlp.workspace_bytes(512))
    x512 = torch.zeros((512, L.H), dtype=x.dtype, device=x.device)
    y512 = torch.full_like(x512, 0x1234)
    with pytest.raises(vq.VqmlpError) as e:
        mlp.forward_noalloc(x512, y512)
    assert e.value.status == vq.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y512 == 0x1234).all())


@pytest.mark.parametrize("H,I,T1,T2", [(512, 1024, 24, 9), (256, 704, 8, 1), (1024, 2048, 64, 16)])
def test_noalloc_matches_forward_small(vq, oracle_mod, torch_dev, H, I, T1, T2):
    torch = torch_dev
    L = synth.mlp_layer(H, I, T1, seed=H + I + T1, outliers=True)
    mlp = vq.MLP.from_layer(L, t_max=T1)
    x = vq.to_device(L.x)
    _say("no-alloc H=%d I=%d T=%d then T=%d" % (H, I, T1, T2))
    y_ref, y = _pair(vq, torch, mlp, x)
    assert torch.equal(y, y_ref)
    got = y.cpu().numpy().view(np.float16).astype(np.float64)
    ref = oracle_mod.mlp_forward(L)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 2e-3
    x2 = x[:T2].clone()
    y_ref2, y2 = _pair(vq, torch, mlp, x2)
    assert torch.equal(y2, y_ref2)


def test_noalloc_matches_forward_vq2(vq, oracle_mod, torch_dev):
    """A 2x16 MLP plan through the allocation-free entry: the T <= 8 projection path, then the
    tiled path (T = 16), then a smaller T <= 8 call again."""
    torch = torch_dev
    L = synth.vq2_mlp_layer(512, 1024, 16, seed=31, outliers=True)
    mlp = vq.MLP.from_vq2_layer(L, t_max=16)
    x = vq.to_device(L.x)
    ref = oracle_mod.vq2_mlp_forward(L)
    for T in (8, 16, 3):
        _say("no-alloc 2x16 T=%d" % T)
        y_ref, y = _pair(vq, torch, mlp, x[:T].clone())
        assert torch.equal(y, y_ref)
        got = y.cpu().numpy().view(np.float16).astype(np.float64)
        assert np.linalg.norm(got - ref[:T]) / np.linalg.norm(ref[:T]) <= 2e-3
