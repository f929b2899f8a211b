"""GPU: VQMLP_TRACE names the kernels that each call's dispatch chose (one stderr line per call),
and nothing is logged when it is unset or "0"."""
import numpy as np
import pytest

from bit_vector_lut_amd import synth

pytestmark = pytest.mark.gpu


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


def _lines(capfd):
    return [l for l in capfd.readouterr().err.splitlines() if l.startswith("vqmlp: ")]


@pytest.mark.parametrize("T,path,want", [
    (1, 0, "fused kernel"), (8, 0, "fused kernel"), (8, 2, "tiled gate/up"),
    (16, 0, "tiled gate/up"), (48, 0, "register-decode gate/up"),
])
def test_trace_mlp_dispatch(vq, torch_dev, capfd, monkeypatch, T, path, want):
    layer = synth.mlp_layer(1024, 2048, T, seed=T)
    mlp = vq.MLP.from_layer(layer, t_max=max(T, 8))
    x = vq.to_device(layer.x)
    capfd.readouterr()
    monkeypatch.setenv("VQMLP_TRACE", "1")
    mlp.forward(x, path=path)
    torch_dev.cuda.synchronize()
    lines = _lines(capfd)
    print("\n".join(lines))
    assert len(lines) == 1, lines
    assert lines[0].startswith("vqmlp: forward H=1024 I=2048 T=%d: " % T), lines
    assert want in lines[0], lines
    monkeypatch.setenv("VQMLP_TRACE", "0")
    mlp.forward(x, path=path)
    torch_dev.cuda.synchronize()
    assert _lines(capfd) == []


def test_trace_vq2_and_lut_dispatch(vq, torch_dev, capfd, monkeypatch):
    layer = synth.vq2_mlp_layer(1024, 2048, 8, seed=3)
    mlp = vq.MLP.from_vq2_layer(layer, t_max=8)
    rng = np.random.default_rng(5)
    lut = vq.LUTProjection.from_proj(synth.lut_projection(rng, 2, 1024, 2048, 64, 1024))
    head = vq.LUTProjection.from_proj(synth.lut_projection(rng, 4, 4096, 1024, 0, 0))
    x8 = vq.to_device(rng.standard_normal((8, 2048)).astype(np.float16))
    x48 = vq.to_device(rng.standard_normal((48, 2048)).astype(np.float16))
    xh = vq.to_device(rng.standard_normal((8, 1024)).astype(np.float16))
    xm = vq.to_device(layer.x)
    capfd.readouterr()
    monkeypatch.setenv("VQMLP_TRACE", "1")
    mlp.forward(xm)
    lut.forward(x8)
    lut.forward(x48)
    head.argmax(xh)
    torch_dev.cuda.synchronize()
    lines = _lines(capfd)
    print("\n".join(lines))
    assert len(lines) == 4, lines
    assert "forward 2x16 H=1024 I=2048 T=8: " in lines[0] and "2x16 projection kernel" in lines[0]
    assert "scalar-LUT 2-bit N=1024 K=2048 T=8 r=64: " in lines[1] and "code-stream" in lines[1]
    assert "scalar-LUT 2-bit N=1024 K=2048 T=48 r=64: " in lines[2]
    assert "register-decode LUT product" in lines[2]
    assert "argmax head 4-bit N=4096 K=1024 T=8: " in lines[3]
    monkeypatch.delenv("VQMLP_TRACE")
    lut.forward(x8)
    torch_dev.cuda.synchronize()
    assert _lines(capfd) == []
