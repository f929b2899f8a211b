"""GPU parity: the HIP library against the FP64 oracle on identical seeded inputs.

Bars: dequantised weights bit-exact; rotation within 1e-6 relative; MLP and scalar-LUT
projection outputs within a relative Frobenius error of 2e-3 (FP32 accumulation and FP16
operands against FP64).
Every call goes through the C ABI (the ctypes binding only marshals arguments).
"""
import sys

import numpy as np
import pytest

from bit_vector_lut_amd import synth

pytestmark = pytest.mark.gpu

MLP_TOL = 2e-3


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


def _f64(t):
    return t.cpu().numpy().view(np.float16).astype(np.float64)


def _rel_fro(y, ref):
    return np.linalg.norm(y - ref) / np.linalg.norm(ref)


ROW_TOL = 1e-2   # worst row (token): relative error of that row
ELEM_TOL = 1e-2  # worst element, relative to the largest |reference| of its row


def _report(name, y, ref, row_scale="own"):
    """Relative Frobenius error (returned), after asserting the local bounds: no row of y and no
    single element may be off by more than 1% of its row's scale, so an error confined to a few
    rows or one tile cannot hide under the whole-matrix norm.  row_scale="global" measures every
    row against the largest row norm instead (for closed forms whose rows can cancel to nearly
    zero, where a row's own norm says nothing about the kernel's accuracy)."""
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), "%s: non-finite outputs" % name
    err = _rel_fro(y, ref)
    rnorm = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    rmax = np.maximum(np.abs(ref).max(axis=1, keepdims=True), 1e-30)
    if row_scale == "global":
        rnorm = np.full_like(rnorm, rnorm.max())
        rmax = np.full_like(rmax, rmax.max())
    row = np.linalg.norm(y - ref, axis=1) / rnorm
    elem = (np.abs(y - ref) / rmax).max()
    _say("%s: rel_fro=%.3e max_abs=%.3e worst_row=%.3e worst_elem=%.3e" % (
        name, err, np.abs(y - ref).max(), row.max(), elem))
    assert row.max() <= ROW_TOL, "%s: worst row %.3e (row %d)" % (name, row.max(), row.argmax())
    assert elem <= ELEM_TOL, "%s: worst element %.3e of its row's scale" % (name, elem)
    return err


# ------------------------------------------------------------------ dequantisation


@pytest.mark.parametrize("N,K", [(32, 64), (64, 256), (704, 256), (256, 704), (96, 128)])
def test_dequant_bit_exact(vq, oracle_mod, torch_dev, N, K):
    m = synth.vq3_matrix(np.random.default_rng(N * 7 + K), N, K)
    # force a few subnormal and signed-zero centroids into play
    cb = m.cb.copy()
    cb.view(np.uint16)[0, :4, 0] = [0x0001, 0x8003, 0x03FF, 0x8000]
    m = synth.VQ3Matrix(m.codes, cb, m.sc)
    _say("dequant N=%d K=%d" % (N, K))
    w = vq.dequant(N, K, vq.to_device(vq.pack(*m.as_u16()))).cpu().numpy()
    ref = oracle_mod.vq3_weight(m.codes, m.cb, m.sc).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_dequant_full_size_row_blocks(vq, oracle_mod, torch_dev):
    """The 27B-like down matrix (5120 x 17408): sampled 32-row blocks, bit-exact."""
    rng = np.random.default_rng(3)
    N, K = 5120, 17408
    m = synth.vq3_matrix(rng, N, K)
    _say("dequant full 5120x17408")
    w = vq.dequant(N, K, vq.to_device(vq.pack(*m.as_u16())))
    for r0 in (0, 2048, 5088):
        sub = synth.VQ3Matrix(m.codes[r0 // 2:r0 // 2 + 16], m.cb[r0 // 8:r0 // 8 + 4],
                              m.sc[r0:r0 + 32])
        ref = oracle_mod.vq3_weight(sub.codes, sub.cb, sub.sc).astype(np.float32)
        got = w[r0:r0 + 32].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), r0


# ------------------------------------------------------------------ rotation


@pytest.mark.parametrize("T,n,b", [(1, 256, 128), (3, 704, 64), (8, 5120, 128), (13, 2048, 1024),
                                   (2, 64, 2), (9, 17408, 128)])
def test_rotate_matches_oracle(vq, oracle_mod, torch_dev, T, n, b):
    rng = np.random.default_rng(T * n + b)
    x = rng.standard_normal((T, n)).astype(np.float16)
    s = rng.lognormal(0, 0.3, n).astype(np.float16)
    sign = (2 * rng.integers(0, 2, n) - 1).astype(np.int8)
    _say("rotate T=%d n=%d b=%d" % (T, n, b))
    got = vq.rotate(vq.to_device(x), b, vq.to_device(s), vq.to_device(sign)).cpu().numpy()
    ref = oracle_mod.rotate(x.astype(np.float64) * s.astype(np.float64), b, sign)
    assert _rel_fro(got.astype(np.float64), ref) <= 1e-6
    assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max() * 4


# ------------------------------------------------------------------ MLP forward


def _run(vq, torch_dev, layer, path=0, mlp=None):
    mlp = mlp or vq.MLP.from_layer(layer, t_max=max(layer.T, 8))
    x = vq.to_device(layer.x)
    y = mlp.forward(x, path=path)
    torch_dev.cuda.synchronize()
    return _f64(y)


@pytest.mark.parametrize("path", [0, 1, 2])
def test_tiny_layer(vq, oracle_mod, torch_dev, path):
    L = synth.tiny_layer()
    _say("tiny_layer path=%d" % path)
    y = _run(vq, torch_dev, L, path)
    ref = oracle_mod.mlp_forward(L)
    assert _report("tiny_layer path %d" % path, y, ref) <= MLP_TOL


SMALL = [(256, 704), (128, 192), (512, 1024), (320, 640)]


@pytest.mark.parametrize("T", [1, 2, 7, 8, 9, 16, 33, 64, 65, 130, 300])
@pytest.mark.parametrize("H,I", SMALL)
def test_mlp_small_shapes(vq, oracle_mod, torch_dev, H, I, T):
    L = synth.mlp_layer(H, I, T, seed=H * 31 + I + T, outliers=(T % 2 == 1))
    _say("small H=%d I=%d T=%d" % (H, I, T))
    mlp = vq.MLP.from_layer(L, t_max=max(T, 8))
    ref = oracle_mod.mlp_forward(L)
    for path in ([0, 1, 2] if T <= 8 else [0]):
        y = _run(vq, torch_dev, L, path, mlp)
        assert _report("H=%d I=%d T=%d path %d" % (H, I, T, path), y, ref) <= MLP_TOL


@pytest.fixture(scope="module")
def layer27b_t8():
    return synth.layer27b_t8()


@pytest.fixture(scope="module")
def layer27b_t8_ref(oracle_mod, layer27b_t8):
    return oracle_mod.mlp_forward(layer27b_t8)


def test_layer27b_t8_full(vq, oracle_mod, torch_dev, layer27b_t8, layer27b_t8_ref):
    _say("layer27b_t8 fused")
    y = _run(vq, torch_dev, layer27b_t8, 0)
    assert _report("layer27b_t8", y, layer27b_t8_ref) <= MLP_TOL


def test_layer27b_t8_tiled_path(vq, oracle_mod, torch_dev, layer27b_t8, layer27b_t8_ref):
    _say("layer27b_t8 tiled")
    y = _run(vq, torch_dev, layer27b_t8, 2)
    assert _report("layer27b_t8 tiled", y, layer27b_t8_ref) <= MLP_TOL


@pytest.mark.parametrize("H,I,T", [(256, 17408, 8), (5120, 1024, 3), (512, 256, 8), (64, 65536, 8),
                                   (1024, 4352, 1), (4096, 1024, 8)])
def test_fused_unusual_shapes(vq, oracle_mod, torch_dev, H, I, T):
    """The fused kernel on shapes far from the 27B-like one: long K with few rows, H larger than
    I (down items then cover more row tiles than I has: nothing of theirs may index I-sized
    arrays by an H row tile), K = 64 with more row tiles than compute units, and T = 1."""
    L = synth.mlp_layer(H, I, T, seed=H + 3 * I + T, outliers=True)
    _say("fused H=%d I=%d T=%d" % (H, I, T))
    mlp = vq.MLP.from_layer(L, t_max=8)
    ref = oracle_mod.mlp_forward(L)
    for path in (0, 1):
        y = _run(vq, torch_dev, L, path, mlp)
        assert _report("fused H=%d I=%d T=%d path %d" % (H, I, T, path), y, ref) <= MLP_TOL


@pytest.mark.parametrize("H,I,T,bh", [(512, 1024, 8, 32), (512, 1024, 3, 64), (512, 1024, 8, 256),
                                       (320, 640, 5, 64), (1024, 2048, 8, 128)])
def test_fused_input_rotation_blocks(vq, oracle_mod, torch_dev, H, I, T, bh):
    """The fused kernel rotates x inside every workgroup, one 64-, 128- or 256-column chunk of
    all 8 operand rows per wave: Hadamard blocks smaller than, and as wide as, the chunk."""
    L = synth.mlp_layer(H, I, T, seed=H + 7 * bh + T, outliers=True, had_block_h=bh)
    _say("fused input rotation H=%d I=%d T=%d bh=%d" % (H, I, T, bh))
    mlp = vq.MLP.from_layer(L, t_max=8)
    ref = oracle_mod.mlp_forward(L)
    y = _run(vq, torch_dev, L, 1, mlp)
    assert _report("bh=%d" % bh, y, ref) <= MLP_TOL


def test_fused_control_block_is_left_ready(vq, oracle_mod, torch_dev):
    """Several fused calls on one workspace (mixed with tiled calls): every call is right, the
    queue and counters are back at zero, the error word stays clear (read through the C ABI),
    the epoch counts calls."""
    L = synth.mlp_layer(512, 1024, 8, seed=11, outliers=True)
    mlp = vq.MLP.from_layer(L, t_max=8)
    x = vq.to_device(L.x)
    ws = mlp.workspace(8)
    ref = oracle_mod.mlp_forward(L)
    fused_calls = 0
    for path in (1, 0, 2, 1, 2, 2, 1, 0, 1):
        _say("control block: path %d" % path)
        y = _f64(mlp.forward(x, workspace=ws, path=path))
        torch_dev.cuda.synchronize()
        assert _report("path %d" % path, y, ref) <= MLP_TOL
        fused_calls += path in (0, 1)  # path 0 takes the fused kernel at T <= 8
    assert vq.workspace_errors(ws, clear=False) == 0
    ctl = ws[:64].cpu().numpy().view(np.uint32)
    assert ctl[0] == 0 and ctl[1] == 0, ctl[:4]  # queue head, exit count
    assert ctl[2] == 0, "a bounded wait ran out: error bits %#x" % ctl[2]
    assert ctl[3] == fused_calls
    assert not ctl[4:].any(), ctl  # the rest of the block is never written


def test_workspace_errors_reads_and_clears(vq, torch_dev):
    """The error word is the third word of the control block: what the call reports is that
    word, and clearing zeroes only that word (written here from the host: a kernel never sets
    it when its waits end normally)."""
    L = synth.mlp_layer(256, 704, 4, seed=2)
    mlp = vq.MLP.from_layer(L, t_max=8)
    ws = mlp.workspace(8)
    mlp.forward(vq.to_device(L.x), workspace=ws)
    assert vq.workspace_errors(ws) == 0
    ws[8:12] = torch_dev.tensor([5, 0, 0, 0], dtype=torch_dev.uint8)
    epoch = ws[12:16].clone()
    assert vq.workspace_errors(ws, clear=False) == 5
    assert vq.workspace_errors(ws) == 5
    assert vq.workspace_errors(ws) == 0
    assert torch_dev.equal(ws[12:16], epoch)
    with pytest.raises(vq.VqmlpError) as e:
        vq.workspace_errors(ws[:32])
    assert e.value.status == vq.ERR_INVALID_ARG


@pytest.mark.parametrize("path", [1, 2])
def test_layer27b_t8_deterministic(vq, torch_dev, layer27b_t8, path):
    mlp = vq.MLP.from_layer(layer27b_t8)
    x = vq.to_device(layer27b_t8.x)
    ws = mlp.workspace(8)
    _say("layer27b_t8 determinism path %d" % path)
    y1 = mlp.forward(x, workspace=ws, path=path).clone()
    y2 = mlp.forward(x, workspace=ws, path=path).clone()
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2)


def test_layer27b_t64_all_tokens(vq, oracle_mod, torch_dev):
    """The 27B-like layer at T = 64 (the fixed prefill chunk), every output."""
    L = synth.layer27b_t64()
    _say("layer27b_t64 T=64")
    mlp = vq.MLP.from_layer(L, t_max=64)
    x = vq.to_device(L.x)
    ws = mlp.workspace(64)
    y1 = mlp.forward(x, workspace=ws)
    y2 = mlp.forward(x, workspace=ws).clone()
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2), "T=64 forward is not bitwise repeatable"
    ref = oracle_mod.mlp_forward(L)
    assert _report("layer27b_t64", _f64(y1), ref) <= MLP_TOL


def test_errors_on_device(vq, torch_dev):
    L = synth.mlp_layer(256, 704, 4, seed=1)
    mlp = vq.MLP.from_layer(L, t_max=8)
    x = vq.to_device(L.x)
    small = torch_dev.zeros(256, dtype=torch_dev.uint8, device="cuda")
    with pytest.raises(vq.VqmlpError) as e:
        mlp.forward(x, workspace=small)
    assert e.value.status == vq.ERR_WORKSPACE
    big = vq.to_device(np.zeros((9, 256), np.float16))
    with pytest.raises(vq.VqmlpError) as e:
        mlp.forward(big)
    assert e.value.status == vq.ERR_INVALID_ARG
    with pytest.raises(vq.VqmlpError) as e:
        mlp.forward(vq.to_device(np.zeros((9, 256), np.float16)), path=1)
    for bad in (3, 4, 5, -1):
        with pytest.raises(vq.VqmlpError) as e:
            mlp.forward(x, path=bad)
        assert e.value.status == vq.ERR_INVALID_ARG
    empty = vq.to_device(np.zeros((0, 256), np.float16))
    assert mlp.forward(empty).shape == (0, 256)


@pytest.fixture(scope="module")
def prefill512():
    return synth.prefill512()


def test_prefill512_mlp_all_tokens(vq, oracle_mod, torch_dev, prefill512):
    """The 27B-like layer at T = 512 (register-decode matrix-core products, K-split down
    projection), every output; a second call is bitwise identical."""
    L = prefill512[0]
    _say("prefill512 MLP T=512")
    mlp = vq.MLP.from_layer(L, t_max=512)
    x = vq.to_device(L.x)
    ws = mlp.workspace(512)
    y1 = mlp.forward(x, workspace=ws)
    y2 = mlp.forward(x, workspace=ws).clone()
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2), "T=512 forward is not bitwise repeatable"
    ref = oracle_mod.mlp_forward(L)
    assert _report("prefill512 MLP", _f64(y1), ref) <= MLP_TOL


@pytest.mark.parametrize("H,I,T,bi", [(1024, 4352, 1024, None), (1024, 4352, 1024, 64),
                                       (5120, 17408, 130, None)])
def test_gateup_leftover_split(vq, oracle_mod, torch_dev, H, I, T, bi):
    """Shapes whose gate/up tiles leave a partial round on 256 CUs: the leftover rows go through
    the K-split product and the combine pass (with the fused 128-row rotation, or with the
    FP32 product and the separate 64-wide rotation)."""
    L = synth.mlp_layer(H, I, T, seed=H + I + T, outliers=True, had_block_i=bi)
    _say("gate/up leftover split H=%d I=%d T=%d bi=%s" % (H, I, T, bi))
    mlp = vq.MLP.from_layer(L, t_max=T)
    y = _run(vq, torch_dev, L, 0, mlp)
    ref = oracle_mod.mlp_forward(L)
    assert _report("leftover split H=%d I=%d T=%d" % (H, I, T), y, ref) <= MLP_TOL


# ------------------------------------------------------------------ scalar-LUT projection

LUT_CASES = [  # N, K, T, rank, Hadamard block (0 = none)
    (64, 1024, 1, 64, 1024),
    (192, 2048, 9, 40, 1024),
    (256, 1024, 65, 64, 256),
    (128, 512, 130, 0, 0),
    (320, 2048, 33, 128, 512),
    (64, 64, 3, 64, 64),
]


LUT8_CASES = [  # decode-size T: the code-stream kernel (K <= 5120), and K past it (tiled)
    (5120, 5120, 8, 64, 1024),  # the token-mixer shape at T = 8
    (192, 320, 5, 0, 64),       # fewer 64-column units than K slices
    (256, 2048, 2, 128, 512),
    (64, 5184, 8, 64, 64),      # K > 5120: tiled kernels
    (128, 1024, 4, 20, 1024),   # rank not a multiple of 8: tiled kernels
    (64, 1024, 7, 256, 256),    # largest rank
    (128, 512, 6, 32, 0),       # no rotation
    (128, 768, 8, 32, 256),     # 256-column chunks (4 columns per lane in the pre-pass)
    (64, 384, 4, 16, 128),      # 128-column chunks (2 columns per lane)
]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("N,K,T,rank,hb", LUT8_CASES)
def test_lut_decode_shapes(vq, oracle_mod, torch_dev, bits, N, K, T, rank, hb):
    """Scalar-LUT projections at T <= 8 against the oracle, every output."""
    rng = np.random.default_rng(N + 5 * K + 11 * T + bits)
    p = synth.lut_projection(rng, bits, N, K, rank, hb)
    x = synth.activations(rng, T, K, outliers=True)
    _say("LUT T<=8 bits=%d N=%d K=%d T=%d r=%d hb=%d" % (bits, N, K, T, rank, hb))
    proj = vq.LUTProjection.from_proj(p)
    xd = vq.to_device(x)
    ws = proj.workspace(T)
    y1 = proj.forward(xd, workspace=ws)
    y2 = proj.forward(xd, workspace=ws).clone()
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2), "not bitwise repeatable"
    ref = oracle_mod.lut_forward(p, x)
    assert _report("LUT T<=8 %d-bit %dx%d T=%d" % (bits, N, K, T), _f64(y1), ref) <= MLP_TOL


HEAD_CASES = [  # N, K, T, Hadamard block (0 = none), bits
    (4096, 5120, 8, 0, 4),
    (1024, 5120, 3, 1024, 4),
    (2048, 512, 1, 0, 2),
    (64, 128, 8, 64, 4),  # fewer 32-row blocks than workgroups
]


@pytest.mark.parametrize("N,K,T,hb,bits", HEAD_CASES)
def test_lut_argmax_head(vq, oracle_mod, torch_dev, N, K, T, hb, bits):
    """Greedy argmax head against the oracle's FP64 logits: the returned row holds the largest
    logit up to the FP32-versus-FP64 accumulation difference (rows whose logits differ by less
    may be ordered either way), and its value is that row's logit."""
    rng = np.random.default_rng(N + K + T + hb + bits)
    p = synth.lut_projection(rng, bits, N, K, 0, hb)
    x = synth.activations(rng, T, K, outliers=True)
    _say("argmax head N=%d K=%d T=%d hb=%d bits=%d" % (N, K, T, hb, bits))
    proj = vq.LUTProjection.from_proj(p)
    xd = vq.to_device(x)
    ws = proj.workspace(T)
    idx, val = proj.argmax(xd, ws)
    idx2, val2 = proj.argmax(xd, ws)
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(idx, idx2) and torch_dev.equal(val, val2), "not bitwise repeatable"
    idx, val = idx.cpu().numpy(), val.cpu().numpy().astype(np.float64)
    assert idx.shape == (T,) and ((idx >= 0) & (idx < N)).all(), idx
    y = oracle_mod.lut_forward(p, x)
    ref_idx, ref_val = oracle_mod.lut_argmax(p, x)
    tol = 2e-3 * np.abs(y).max(axis=1)
    for t in range(T):
        assert y[t, idx[t]] >= ref_val[t] - tol[t], (t, idx[t], ref_idx[t])
        assert abs(val[t] - y[t, idx[t]]) <= tol[t]


def test_lut_argmax_full_head_planted(vq, torch_dev):
    """The 248,320-row four-bit output head at T = 8 (property test: no oracle pass over 1.3 G
    weights).  Token t's x is positive on its own 640 columns and zero elsewhere; row planted[t]
    takes its table's entry 15 (= 1) on those columns and entry 0 (= 0) elsewhere, so its logit
    for token t is about 640 x sc while every random row stays near 0.02 sqrt(640) and the other
    planted rows give 0: the head must return planted[t] for token t, with that logit."""
    N, K, T = 248320, 5120, 8
    span = K // T
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    lut = (rng.standard_normal((N // 8, 16)) * 0.02).astype(np.float16)
    sc = rng.uniform(0.5, 1.5, N).astype(np.float16)
    planted = rng.choice(N, T, replace=False)
    x = np.zeros((T, K), np.float16)
    for t, j in enumerate(planted):
        cols = slice(t * span, (t + 1) * span)
        x[t, cols] = (np.abs(rng.standard_normal(span)) + 0.1).astype(np.float16)
        lut[j // 8, 15], lut[j // 8, 0] = np.float16(1.0), np.float16(0.0)
        codes[j, :] = 0
        codes[j, cols] = 15
    packed = vq.to_device(vq.lut_pack(4, codes, lut, sc))
    del codes
    proj = vq.LUTProjection(4, N, K, packed, None, None, None, None, 0)
    _say("argmax head full 248320 x 5120 T=8")
    idx, val = proj.argmax(vq.to_device(x))
    torch_dev.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy().astype(np.float64)
    assert ((idx >= 0) & (idx < N)).all(), idx
    assert list(idx) == [int(j) for j in planted]
    for t, j in enumerate(planted):
        want = float(sc[j]) * float(x[t].astype(np.float64).sum())
        assert abs(val[t] - want) <= 1e-3 * want


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("N,K,T,rank,hb", LUT_CASES)
def test_lut_small_shapes(vq, oracle_mod, torch_dev, bits, N, K, T, rank, hb):
    rng = np.random.default_rng(N + 3 * K + 7 * T + bits)
    p = synth.lut_projection(rng, bits, N, K, rank, hb)
    x = rng.standard_normal((T, K)).astype(np.float16)
    _say("lut bits=%d N=%d K=%d T=%d r=%d hb=%d" % (bits, N, K, T, rank, hb))
    proj = vq.LUTProjection.from_proj(p)
    y = _f64(proj.forward(vq.to_device(x)))
    torch_dev.cuda.synchronize()
    ref = oracle_mod.lut_forward(p, x)
    assert _report("lut%d N=%d K=%d T=%d" % (bits, N, K, T), y, ref) <= MLP_TOL


@pytest.mark.parametrize("which", [1, 2])
def test_prefill512_lut_all_tokens(vq, oracle_mod, torch_dev, prefill512, which):
    L, p = prefill512[0], prefill512[which]
    _say("prefill512 lut%d T=512" % p.bits)
    proj = vq.LUTProjection.from_proj(p)
    xd = vq.to_device(L.x)
    ws = proj.workspace(512)
    y1 = proj.forward(xd, workspace=ws)
    y2 = proj.forward(xd, workspace=ws).clone()
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2), "not bitwise repeatable"
    ref = oracle_mod.lut_forward(p, L.x)
    assert _report("prefill512 lut%d" % p.bits, _f64(y1), ref) <= MLP_TOL


def test_lut_errors_on_device(vq, torch_dev):
    rng = np.random.default_rng(5)
    p = synth.lut_projection(rng, 2, 64, 128, 64, 128)
    proj = vq.LUTProjection.from_proj(p)
    x = vq.to_device(rng.standard_normal((4, 128)).astype(np.float16))
    small = torch_dev.zeros(256, dtype=torch_dev.uint8, device="cuda")
    for fwd in (proj.forward, proj.forward_stateless):
        with pytest.raises(vq.VqmlpError) as e:
            fwd(x, workspace=small)
        assert e.value.status == vq.ERR_WORKSPACE
    # a header that does not match (bits) and a block that does not divide K: rejected by the
    # stateless call and by plan creation alike
    args = (proj.packed, proj.U, proj.V, proj.s, proj.sign)
    for bits, hb in ((4, 128), (2, 96)):
        with pytest.raises(vq.VqmlpError) as e:
            vq.LUTProjection(bits, p.N, p.K, *args, had_block=hb)
        assert e.value.status == vq.ERR_INVALID_ARG
        proj.bits, proj.had_block = bits, hb
        with pytest.raises(vq.VqmlpError) as e:
            proj.forward_stateless(x)
        assert e.value.status == vq.ERR_INVALID_ARG
    proj.bits, proj.had_block = 2, 128
    empty = vq.to_device(np.zeros((0, 128), np.float16))
    assert proj.forward(empty).shape == (0, 64)
    assert proj.forward_stateless(empty).shape == (0, 64)
    # the plan and the stateless call give the same bits
    y1, y2 = proj.forward(x), proj.forward_stateless(x)
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2)


VQ2_CASES = [  # N, K, T
    (32, 32, 1),        # one tile, one 32-column unit: 15 of 16 slices empty
    (64, 96, 5),        # ragged slices
    (160, 320, 8),
    (5120, 5120, 8),    # the previous format's down-projection output width
    (17408, 5120, 7),   # gate / up shape
]


@pytest.mark.gpu
@pytest.mark.parametrize("N,K,T", VQ2_CASES)
def test_vq2_projection(vq, oracle_mod, torch_dev, N, K, T):
    """2x16 vector-LUT projection at T <= 8 against the oracle's FP64 product, every output."""
    rng = np.random.default_rng(N + 3 * K + T)
    m = synth.vq2_matrix(rng, N, K)
    x = synth.activations(rng, T, K, outliers=True)
    _say("2x16 projection N=%d K=%d T=%d" % (N, K, T))
    proj = vq.VQ2Projection.from_matrix(m)
    xd = vq.to_device(x)
    y1 = proj.forward(xd)
    y2 = proj.forward(xd)
    torch_dev.cuda.synchronize()
    assert torch_dev.equal(y1, y2), "not bitwise repeatable"
    y = _f64(y1)
    ref = oracle_mod.vq2_matmul(m.codes, m.cb, m.sc, x)
    assert _report("2x16 %dx%d T=%d" % (N, K, T), y, ref) <= MLP_TOL


@pytest.mark.gpu
def test_vq2_projection_limits(vq, torch_dev):
    m = synth.vq2_matrix(np.random.default_rng(9), 64, 64)
    proj = vq.VQ2Projection.from_matrix(m)
    x = vq.to_device(np.zeros((9, 64), np.float16))
    with pytest.raises(vq.VqmlpError, match="T <= 8"):
        proj.forward(x)
    big = synth.vq2_matrix(np.random.default_rng(10), 32, 5152)
    with pytest.raises(vq.VqmlpError, match="above 5120"):
        vq.VQ2Projection.from_matrix(big)


@pytest.mark.gpu
def test_vq2_and_argmax_t0_noop(vq, torch_dev):
    """T == 0 launches nothing and leaves the outputs untouched."""
    torch = torch_dev
    m = synth.vq2_matrix(np.random.default_rng(21), 64, 64)
    proj = vq.VQ2Projection.from_matrix(m)
    y = torch.full((0, 64), 7, dtype=torch.int16, device="cuda")
    proj.forward(vq.to_device(np.zeros((0, 64), np.float16)), y)
    head = vq.LUTProjection.from_proj(synth.lut_projection(np.random.default_rng(22), 4, 64, 64, 0, 0))
    idx, val = head.argmax(vq.to_device(np.zeros((0, 64), np.float16)), head.workspace(8))
    torch.cuda.synchronize()
    assert idx.numel() == 0 and val.numel() == 0


@pytest.mark.gpu
def test_vq2_and_argmax_graph_replays_match_eager(vq, torch_dev):
    """The 2x16 projection and the argmax head captured in one HIP graph: every replay (with
    eager work and synchronisations between them) reproduces the eager results bit for bit."""
    torch = torch_dev
    rng = np.random.default_rng(23)
    proj = vq.VQ2Projection.from_matrix(synth.vq2_matrix(rng, 1024, 512))
    head = vq.LUTProjection.from_proj(synth.lut_projection(rng, 4, 2048, 512, 0, 0))
    x = vq.to_device(synth.activations(rng, 8, 512, True))
    ws = head.workspace(8)
    st = torch.cuda.Stream()
    y = torch.empty((8, 1024), dtype=x.dtype, device="cuda")
    with torch.cuda.stream(st):
        proj.forward(x, y, stream=st)
        idx, val = head.argmax(x, ws, stream=st)
    st.synchronize()
    ref = (y.clone(), idx.clone(), val.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        proj.forward(x, y, stream=st)
        gi, gv = head.argmax(x, ws, stream=st)
    for rep in range(3):
        y.zero_()
        gi.fill_(-1)
        gv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]), "replay %d: 2x16 output" % rep
        assert torch.equal(gi, ref[1]) and torch.equal(gv, ref[2]), "replay %d: argmax" % rep


# ------------------------------------------------------------------ closed forms on the GPU


def _blockdiag_rotation(u, b, sign):
    """(I (x) H_b / sqrt(b)) diag(sign) applied to the rows of u, from scipy's Sylvester matrix."""
    import scipy.linalg

    Hb = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    v = u * sign.astype(np.float64)[None, :]
    T, n = v.shape
    return (v.reshape(T, n // b, b) @ Hb.T).reshape(T, n)


def _identity_vq3(n):
    """W = I: entry 1 = (1, 0), entry 2 = (0, 1), everything else (0, 0); unit scales."""
    cb = np.zeros((n // 8, 64, 2), np.float16)
    cb[:, 1, 0] = 1
    cb[:, 2, 1] = 1
    codes = np.zeros((n // 2, n), np.uint8)
    p = np.arange(n // 2)
    codes[p, 2 * p] = 1
    codes[p, 2 * p + 1] = 2
    return synth.VQ3Matrix(codes, cb, np.ones(n, np.float16))


@pytest.mark.parametrize("T", [1, 8, 64, 130])
def test_identity_weights_closed_form(vq, torch_dev, T):
    """Gate = up = down = I (exactly representable): y = R_I(silu(x~) x~) with x~ = R_H(x s), the
    rotations built from scipy's Hadamard matrix: the kernels' decode, products, epilogue and
    both rotations against the definition, with no oracle in between."""
    import scipy.special

    n = 1024
    L = synth.mlp_layer(n, n, T, seed=40 + T, outliers=False)
    L.gate = L.up = L.down = _identity_vq3(n)
    _say("identity weights T=%d" % T)
    y = _run(vq, torch_dev, L, 0, vq.MLP.from_layer(L, t_max=max(T, 8)))
    xt = _blockdiag_rotation(L.x.astype(np.float64) * L.s.astype(np.float64), 128, L.sign_h)
    expect = _blockdiag_rotation(xt * scipy.special.expit(xt) * xt, 128, L.sign_i)
    assert _report("identity T=%d" % T, y, expect) <= MLP_TOL


@pytest.mark.parametrize("T", [2, 8, 64, 96])
def test_constant_codebooks_closed_form(vq, torch_dev, T):
    """Every centroid of gate, up and down is (c, c): each projection output is its row scale
    times c times the sum of its input, and the sum of a rotated row is sqrt(b) times the sum of
    the first (signed) entry of each block (the first Hadamard column is the only one that does
    not sum to zero).  So y[t][h] = c_d sc_d[h] sqrt(b_I) sum_B d_I[Bb] a[t][Bb] with a = silu(g) v,
    g[t][r] = c_g sc_g[r] S_t, v[t][r] = c_u sc_u[r] S_t, S_t = sqrt(b_H) sum_B d_H[Bb] u[t][Bb]."""
    import scipy.special

    H, I = 1024, 2048
    L = synth.mlp_layer(H, I, T, seed=50 + T, outliers=False)
    cg, cu, cd = 0.375, -0.25, 0.125
    L.gate = synth.VQ3Matrix(L.gate.codes, np.full((I // 8, 64, 2), cg, np.float16), L.gate.sc)
    L.up = synth.VQ3Matrix(L.up.codes, np.full((I // 8, 64, 2), cu, np.float16), L.up.sc)
    L.down = synth.VQ3Matrix(L.down.codes, np.full((H // 8, 64, 2), cd, np.float16), L.down.sc)
    _say("constant codebooks T=%d" % T)
    y = _run(vq, torch_dev, L, 0, vq.MLP.from_layer(L, t_max=max(T, 8)))
    bh, bi = L.had_block_h, L.had_block_i
    u = L.x.astype(np.float64) * L.s.astype(np.float64)
    S = np.sqrt(bh) * (u[:, ::bh] * L.sign_h[::bh].astype(np.float64)).sum(axis=1)
    g = cg * L.gate.sc.astype(np.float64)[None, :] * S[:, None]
    v = cu * L.up.sc.astype(np.float64)[None, :] * S[:, None]
    a = g * scipy.special.expit(g) * v
    Sa = np.sqrt(bi) * (a[:, ::bi] * L.sign_i[::bi].astype(np.float64)).sum(axis=1)
    expect = cd * L.down.sc.astype(np.float64)[None, :] * Sa[:, None]
    # a token's outputs all share one factor, a signed sum over the rotation blocks that can
    # nearly cancel: its rows are measured against the largest row
    assert _report("constant T=%d" % T, y, expect, row_scale="global") <= MLP_TOL


@pytest.mark.parametrize("bits", [2, 4])
def test_lut_argmax_ties_pick_lowest_row(vq, torch_dev, bits):
    """Two rows per token with bitwise equal logits (same codes, scale and table entries; x and
    the tables are small integers and powers of two, so every partial sum is exact in FP32 in any
    order): the head must return the lower of the two rows.  The pairs are placed both ways round
    (lower row in an earlier and in a later 32-row block than the other, same block too)."""
    N, K, T = 4096, 1024, 4
    top = (1 << bits) - 1
    span = K // T
    rng = np.random.default_rng(77 + bits)
    codes = rng.integers(0, top + 1, size=(N, K), dtype=np.uint8)
    lut = (rng.standard_normal((N // 8, 1 << bits)) * 0.02).astype(np.float16)
    sc = rng.uniform(0.5, 1.5, N).astype(np.float16)
    pairs = [(3000, 17), (40, 41), (2048, 4095), (1000, 999)]
    x = np.zeros((T, K), np.float16)
    for t, rows in enumerate(pairs):
        cols = slice(t * span, (t + 1) * span)
        x[t, cols] = 1.0
        for j in rows:
            lut[j // 8, top], lut[j // 8, 0] = np.float16(1.0), np.float16(0.0)
            codes[j, :] = 0
            codes[j, cols] = top
            sc[j] = np.float16(1.0)
    # every other row of those groups stays below the planted logit (span): its table entries
    # are 0, 1 or N(0, 0.02) values, and entry 'top' appears on about a (1 / 2^bits) share of
    # the columns only
    packed = vq.to_device(vq.lut_pack(bits, codes, lut, sc))
    proj = vq.LUTProjection(bits, N, K, packed, None, None, None, None, 0)
    _say("argmax ties bits=%d" % bits)
    idx, val = proj.argmax(vq.to_device(x))
    torch_dev.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    assert ((idx >= 0) & (idx < N)).all(), idx
    assert list(idx) == [min(p) for p in pairs], (list(idx), pairs)
    assert np.array_equal(val, np.full(T, float(span), np.float32))


# ------------------------------------------------------------------ 2x16 MLP (previous format)


@pytest.mark.parametrize("T", [1, 3, 8, 9, 33, 64, 130, 300])
@pytest.mark.parametrize("H,I", [(256, 512), (512, 1024), (320, 640), (256, 704)])
def test_vq2_mlp_small_shapes(vq, oracle_mod, torch_dev, H, I, T):
    """The 2x16 MLP against the oracle's composition, every output: the T <= 8 projection path
    (path 1, where I is a multiple of 128) and the tiled path with the 2x16 decoder (path 2)."""
    L = synth.vq2_mlp_layer(H, I, T, seed=H + 5 * I + T, outliers=(T % 2 == 1))
    _say("2x16 MLP H=%d I=%d T=%d" % (H, I, T))
    mlp = vq.MLP.from_vq2_layer(L, t_max=max(T, 8))
    ref = oracle_mod.vq2_mlp_forward(L)
    paths = [0, 2] + ([1] if T <= 8 and I % 128 == 0 else [])
    for path in paths:
        y = _run(vq, torch_dev, L, path, mlp)
        assert _report("2x16 H=%d I=%d T=%d path %d" % (H, I, T, path), y, ref) <= MLP_TOL
    if T <= 8 and I % 128:
        with pytest.raises(vq.VqmlpError) as e:
            mlp.forward(vq.to_device(L.x), path=1)
        assert e.value.status == vq.ERR_UNSUPPORTED


@pytest.mark.parametrize("T,paths", [(8, (0, 2)), (64, (0,))])
def test_vq2_mlp_27b_shape(vq, oracle_mod, torch_dev, T, paths):
    """The 27B-like shape in the 2x16 format (down K = 17408: four K slices on the T <= 8 path),
    every output; repeated calls are bitwise identical."""
    L = synth.vq2_mlp_layer(5120, 17408, T, seed=T, outliers=(T == 8))
    _say("2x16 MLP 27B-like T=%d" % T)
    mlp = vq.MLP.from_vq2_layer(L, t_max=T)
    ref = oracle_mod.vq2_mlp_forward(L)
    x = vq.to_device(L.x)
    ws = mlp.workspace(T)
    for path in paths:
        y1 = mlp.forward(x, workspace=ws, path=path)
        y2 = mlp.forward(x, workspace=ws, path=path).clone()
        torch_dev.cuda.synchronize()
        assert torch_dev.equal(y1, y2), "path %d not bitwise repeatable" % path
        assert _report("2x16 27B-like T=%d path %d" % (T, path), _f64(y1), ref) <= MLP_TOL
