"""Pins of the FP64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked fixtures under
tests/golden/, textbook closed forms, library routines (numpy's binary16 conversion,
scipy.linalg.hadamard, scipy.special.expit, numpy matmul) and invariants that hold exactly.
They are chosen so that a dropped term, a wrong sign, a swapped component or row index, or a
transposed operand in the oracle fails at least one of them.
"""
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special

from bit_vector_lut_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    """Parse 'key = values' lines and bare-key matrix blocks (comments start with '#')."""
    out, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if "=" in line:
                k, v = line.split("=", 1)
                out[k.strip()] = v.strip()
                cur = None
            elif line.replace(" ", "").isalpha():
                cur = line
                out[cur] = []
            else:
                out[cur].append([float(t) for t in line.split()])
    return out


# ------------------------------------------------------------------------------ binary16


def test_f16_decode_all_patterns(oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle_mod.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("bits,val", [(0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24),
                                      (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14),
                                      (0x7BFF, 65504.0), (0x3555, 0.333251953125)])
def test_f16_decode_textbook_values(oracle_mod, bits, val):
    assert oracle_mod.f16_to_f64(np.array([bits], np.uint16))[0] == val


# ------------------------------------------------------------------------------ Hadamard


@pytest.mark.parametrize("b", [1 << k for k in range(11)])
def test_hadamard_orthogonal_integer(oracle_mod, b):
    H = oracle_mod.hadamard(b).astype(np.int64)
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=np.int64))


@pytest.mark.parametrize("b", [1 << k for k in range(11)])
def test_hadamard_is_sylvester(oracle_mod, b):
    assert np.array_equal(oracle_mod.hadamard(b), scipy.linalg.hadamard(b))


def test_hadamard4_golden_and_worked_rotation(oracle_mod):
    g = _read_golden("hadamard4.txt")
    H4 = np.array(g["H"], dtype=np.int8)
    assert np.array_equal(oracle_mod.hadamard(4), H4)
    rotated = np.array([float(t) for t in g["rotated"].split()])
    got = oracle_mod.rotate(np.array([[1.0, 2.0, 3.0, 4.0]]), 4, np.array([1, -1, 1, 1], np.int8))
    assert np.array_equal(got[0], rotated)


def _blockdiag_rotate_ref(u, b, sign=None):
    """Library composition: block-diagonal scipy Hadamard / sqrt(b) applied to sign * u."""
    u = np.atleast_2d(np.asarray(u, np.float64))
    if sign is not None:
        u = u * sign
    Hb = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    R = scipy.linalg.block_diag(*([Hb] * (u.shape[1] // b)))
    return u @ R.T


@pytest.mark.parametrize("n,b", [(256, 128), (704, 64), (64, 1), (96, 32), (2048, 1024)])
def test_rotation_matches_library(oracle_mod, n, b):
    rng = np.random.default_rng(n + b)
    u = rng.standard_normal((3, n))
    sign = (2 * rng.integers(0, 2, n) - 1).astype(np.int8)
    got = oracle_mod.rotate(u, b, sign)
    ref = _blockdiag_rotate_ref(u, b, sign)
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("b", [2, 16, 128, 1024])
def test_rotation_round_trip_and_norm(oracle_mod, b):
    rng = np.random.default_rng(b)
    n = 4 * b
    u = rng.standard_normal((2, n))
    sign = (2 * rng.integers(0, 2, n) - 1).astype(np.int8)
    r = oracle_mod.rotate(u, b, sign)
    # R = H D / sqrt(b) is orthogonal: R^T R u = D H H D u / b = u
    back = oracle_mod.rotate(r, b) * sign
    assert np.max(np.abs(back - u)) <= 1e-13 * np.max(np.abs(u))
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), rtol=1e-14)
    # without signs the Sylvester matrix is symmetric, so R R = I
    twice = oracle_mod.rotate(oracle_mod.rotate(u, b), b)
    assert np.max(np.abs(twice - u)) <= 1e-13 * np.max(np.abs(u))


@pytest.mark.parametrize("b", [4, 128])
def test_rotation_closed_forms(oracle_mod, b):
    # all-ones block -> sqrt(b) * e_0 (every other row of H sums to zero)
    r = oracle_mod.rotate(np.ones((1, 2 * b)), b)[0]
    expect = np.zeros(2 * b)
    expect[0] = expect[b] = np.sqrt(b)
    assert np.allclose(r, expect, atol=1e-12)
    # e_0 -> constant 1/sqrt(b) over its block only
    e0 = np.zeros((1, 2 * b))
    e0[0, 0] = 1
    r = oracle_mod.rotate(e0, b)[0]
    assert np.allclose(r[:b], 1 / np.sqrt(b)) and np.all(r[b:] == 0)


# ------------------------------------------------------------------------------ SiLU


def test_silu_matches_tanh_form_and_expit(oracle_mod):
    g = np.concatenate([np.linspace(-40, 40, 4001), [0.0, 1e-8, -1e-8, 1e-300]])
    got = oracle_mod.silu(g)
    tanh_form = 0.5 * g * (1 + np.tanh(g / 2))  # the pages' stated identity
    # (1 + tanh) cancels in FP64 for large negative g, so compare that form where it is accurate
    ok = g > -5
    assert np.allclose(got[ok], tanh_form[ok], rtol=1e-12, atol=1e-300)
    assert np.all(np.abs(got[~ok] - tanh_form[~ok]) <= 1e-5)
    assert np.allclose(got, g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    assert got[g == 0.0][0] == 0.0
    assert oracle_mod.silu(np.array([50.0]))[0] == pytest.approx(50.0, rel=1e-20)


# ------------------------------------------------------------------------------ VQ3 dequantisation


def _golden_vq3():
    g = _read_golden("vq3_two_groups.txt")
    c = np.arange(64, dtype=np.float64)
    cb = np.zeros((2, 64, 2))
    cb[0, :, 0], cb[0, :, 1] = c / 4, -c / 8
    cb[1, :, 0], cb[1, :, 1] = -c / 2, c
    sc = np.array([float(t) for t in g["sc"].split()])
    codes = np.array(g["codes"], dtype=np.uint8)
    W = np.array(g["W"])
    return codes, cb.astype(np.float16), sc.astype(np.float16), W


def test_vq3_golden_hand_worked(oracle_mod):
    codes, cb, sc, W = _golden_vq3()
    assert np.array_equal(oracle_mod.vq3_weight(codes, cb, sc), W)


def test_vq3_golden_matmul(oracle_mod):
    codes, cb, sc, W = _golden_vq3()
    xin = np.array([[1.0, 2.0, -1.0], [0.5, 0.0, 4.0]])
    assert np.array_equal(oracle_mod.vq3_matmul(codes, cb, sc, xin), xin @ W.T)


@pytest.mark.parametrize("N,K,T", [(16, 8, 1), (16, 64, 3), (32, 40, 2)])
def test_vq3_on_the_fly_equals_materialised(oracle_mod, N, K, T):
    rng = np.random.default_rng(N * K + T)
    m = synth.vq3_matrix(rng, N, K)
    xin = rng.standard_normal((T, K))
    W = oracle_mod.vq3_weight(m.codes, m.cb, m.sc)
    got = oracle_mod.vq3_matmul(m.codes, m.cb, m.sc, xin)
    ref = np.matmul(xin, W.T)
    assert np.allclose(got, ref, rtol=0, atol=1e-15 * max(1.0, np.abs(ref).max()))
    # materialised W against numpy indexing of the unpacked arrays (rows 2p / 2p+1, group r//8)
    r = np.arange(N)[:, None]
    j = np.arange(K)[None, :]
    Wn = m.cb.astype(np.float64)[r // 8, m.codes[r // 2, j], r % 2] * m.sc.astype(np.float64)[r]
    assert np.array_equal(W, Wn)


def test_vq3_identity_codebook(oracle_mod):
    # entries 0:(0,0) 1:(1,0) 2:(0,1) with unit scales represent W = I exactly
    n = 16
    cb = np.zeros((n // 8, 64, 2))
    cb[:, 1, 0] = 1
    cb[:, 2, 1] = 1
    codes = np.zeros((n // 2, n), np.uint8)
    for p in range(n // 2):
        codes[p, 2 * p] = 1
        codes[p, 2 * p + 1] = 2
    W = oracle_mod.vq3_weight(codes, cb.astype(np.float16), np.ones(n, np.float16))
    assert np.array_equal(W, np.eye(n))


def test_vq3_codebook_permutation_invariance(oracle_mod):
    rng = np.random.default_rng(7)
    m = synth.vq3_matrix(rng, 32, 24)
    perm = rng.permutation(64)
    inv = np.argsort(perm)
    cb2 = m.cb[:, perm, :]  # new entry e holds old entry perm[e]
    codes2 = inv[m.codes].astype(np.uint8)  # old code c is now at position inv[c]
    assert np.array_equal(oracle_mod.vq3_weight(m.codes, m.cb, m.sc),
                          oracle_mod.vq3_weight(codes2, cb2, m.sc))


def test_vq3_rejects_bad_codes(oracle_mod):
    m = synth.vq3_matrix(np.random.default_rng(1), 8, 4)
    m.codes[0, 0] = 64
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.vq3_weight(m.codes, m.cb, m.sc)


# ------------------------------------------------------------------------------ MLP forward


def _materialise(m):
    N, K = m.N, m.K
    r = np.arange(N)[:, None]
    j = np.arange(K)[None, :]
    return m.cb.astype(np.float64)[r // 8, m.codes[r // 2, j], r % 2] * m.sc.astype(np.float64)[r]


def _mlp_library_composition(L):
    """numpy/scipy FP64 composition: block_diag(hadamard)/sqrt(b), matmul, expit."""
    u = L.x.astype(np.float64) * L.s.astype(np.float64)
    xt = _blockdiag_rotate_ref(u, L.had_block_h, L.sign_h)
    g = xt @ _materialise(L.gate).T
    v = xt @ _materialise(L.up).T
    a = g * scipy.special.expit(g) * v
    at = _blockdiag_rotate_ref(a, L.had_block_i, L.sign_i)
    return at @ _materialise(L.down).T


@pytest.mark.parametrize("H,I,T,outl", [(64, 128, 3, False), (256, 704, 1, False),
                                        (128, 192, 4, True)])
def test_mlp_equals_library_composition(oracle_mod, H, I, T, outl):
    L = synth.mlp_layer(H, I, T, seed=H + I, outliers=outl)
    y = oracle_mod.mlp_forward(L)
    ref = _mlp_library_composition(L)
    assert np.linalg.norm(y - ref) <= 1e-12 * np.linalg.norm(ref)


def test_mlp_identity_weights_closed_form(oracle_mod):
    n = 64
    L = synth.mlp_layer(n, n, 2, seed=3)
    cb = np.zeros((n // 8, 64, 2))
    cb[:, 1, 0] = 1
    cb[:, 2, 1] = 1
    codes = np.zeros((n // 2, n), np.uint8)
    for p in range(n // 2):
        codes[p, 2 * p], codes[p, 2 * p + 1] = 1, 2
    ident = synth.VQ3Matrix(codes, cb.astype(np.float16), np.ones(n, np.float16))
    L.gate = L.up = L.down = ident
    L.had_block_h, L.had_block_i = 32, 64
    y = oracle_mod.mlp_forward(L)
    xt = _blockdiag_rotate_ref(L.x.astype(np.float64) * L.s.astype(np.float64), 32, L.sign_h)
    expect = _blockdiag_rotate_ref(xt * scipy.special.expit(xt) * xt, 64, L.sign_i)
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-14)


def test_mlp_constant_codebook_closed_form(oracle_mod):
    L = synth.mlp_layer(64, 96, 2, seed=5)
    c = 0.375
    L.gate = synth.VQ3Matrix(L.gate.codes, np.full((96 // 8, 64, 2), c, np.float16), L.gate.sc)
    out = oracle_mod.mlp_forward(L, intermediates=True)
    expect = c * L.gate.sc.astype(np.float64)[None, :] * out["xt"].sum(axis=1, keepdims=True)
    assert np.allclose(out["g"], expect, rtol=1e-13, atol=1e-13)


def test_mlp_gated_product_uses_gate_in_silu(oracle_mod):
    L = synth.mlp_layer(64, 96, 3, seed=11)
    out = oracle_mod.mlp_forward(L, intermediates=True)
    g, v = out["g"], out["v"]
    assert np.allclose(out["a"], g * scipy.special.expit(g) * v, rtol=1e-14, atol=0)
    assert not np.allclose(out["a"], v * scipy.special.expit(v) * g, rtol=1e-3)


def test_mlp_down_scale_is_linear(oracle_mod):
    L = synth.mlp_layer(64, 128, 2, seed=9)
    y = oracle_mod.mlp_forward(L)
    L.down = synth.VQ3Matrix(L.down.codes, L.down.cb, (L.down.sc.astype(np.float32) * 2)
                             .astype(np.float16))
    assert np.array_equal(oracle_mod.mlp_forward(L), 2 * y)


def test_mlp_token_independence_and_sign_symmetry(oracle_mod):
    L = synth.mlp_layer(64, 128, 4, seed=13, outliers=True)
    y = oracle_mod.mlp_forward(L)
    assert np.array_equal(oracle_mod.mlp_forward(L, tokens=[2]), y[2:3])
    # negating input channel j and flipping its rotation sign leaves y unchanged (exactly)
    j = np.array([0, 5, 63])
    L.x = L.x.copy()
    L.x[:, j] = -L.x[:, j]
    L.sign_h = L.sign_h.copy()
    L.sign_h[j] = -L.sign_h[j]
    assert np.array_equal(oracle_mod.mlp_forward(L), y)


def test_mlp_codebook_permutation_leaves_output_identical(oracle_mod):
    L = synth.mlp_layer(64, 128, 2, seed=17)
    y = oracle_mod.mlp_forward(L)
    rng = np.random.default_rng(0)
    perm = rng.permutation(64)
    inv = np.argsort(perm)
    d = L.down
    L.down = synth.VQ3Matrix(inv[d.codes].astype(np.uint8), d.cb[:, perm, :], d.sc)
    assert np.array_equal(oracle_mod.mlp_forward(L), y)


# ------------------------------------------------------------------------------ scalar-LUT projection


def test_lut2_golden_hand_worked(oracle_mod):
    g = _read_golden("lut2_tiny.txt")
    lut = np.array([float(t) for t in g["lut"].split()], np.float16)[None, :]
    sc = np.array([float(t) for t in g["sc"].split()], np.float16)
    codes = np.array(g["codes"], np.uint8)
    assert np.array_equal(oracle_mod.lut_weight(2, codes, lut, sc), np.array(g["W"]))


def _lut_library(p, x):
    u = x.astype(np.float64) * (p.s.astype(np.float64) if p.s is not None else 1.0)
    if p.had_block:
        xt = _blockdiag_rotate_ref(u, p.had_block, p.sign)
    else:
        xt = u * (p.sign if p.sign is not None else 1)
    n = np.arange(p.N)[:, None]
    W = p.lut.astype(np.float64)[n // 8, p.codes] * p.sc.astype(np.float64)[:, None]
    y = xt @ W.T
    if p.rank:
        y = y + (xt @ p.V.astype(np.float64).T) @ p.U.astype(np.float64).T
    return y


@pytest.mark.parametrize("bits,b,rank", [(2, 1024, 64), (4, 1024, 8), (4, 0, 0), (2, 64, 0)])
def test_lut_forward_equals_library_composition(oracle_mod, bits, b, rank):
    rng = np.random.default_rng(bits * 100 + rank)
    K = 2048 if b == 1024 else 256
    p = synth.lut_projection(rng, bits, 64, K, rank, b)
    x = rng.standard_normal((3, K)).astype(np.float16)
    y = oracle_mod.lut_forward(p, x)
    ref = _lut_library(p, x)
    assert np.linalg.norm(y - ref) <= 1e-12 * np.linalg.norm(ref)


def test_lut_low_rank_only(oracle_mod):
    rng = np.random.default_rng(2)
    p = synth.lut_projection(rng, 4, 32, 128, 16, 0)
    p.lut = np.zeros_like(p.lut)
    p.s, p.sign = None, None
    x = rng.standard_normal((2, 128)).astype(np.float16)
    y = oracle_mod.lut_forward(p, x)
    ref = (x.astype(np.float64) @ p.V.astype(np.float64).T) @ p.U.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-16)


# ------------------------------------------------------------------------------ output head argmax


def _head(N, K, seed):
    """A 4-bit LUT output head with no rotation or factors (the head's own form)."""
    return synth.lut_projection(np.random.default_rng(seed), 4, N, K, 0, 0)


def test_lut_argmax_planted_maximum_and_ties(oracle_mod):
    p = _head(256, 64, 3)
    p.lut = np.zeros_like(p.lut)
    p.codes = np.zeros_like(p.codes)
    p.s, p.sign = None, None
    p.sc = np.ones_like(p.sc)
    # rows 77 and 140 share the largest logit (their tables' entry 15 = 1, all codes 15); row 13 is
    # half as large; every other logit is 0
    for j, v in ((77, 1.0), (140, 1.0), (13, 0.5)):
        p.lut[j // 8, 15] = v
        p.codes[j, :] = 15
    x = np.ones((3, 64), np.float16)
    x[2] = -1  # all planted logits negative: the largest is 0, first at row 0
    idx, val = oracle_mod.lut_argmax(p, x)
    assert list(idx) == [77, 77, 0]
    assert val[0] == 64.0 and val[2] == 0.0


def test_lut_argmax_equals_brute_force(oracle_mod):
    p = _head(512, 128, 4)
    x = np.random.default_rng(5).standard_normal((8, 128)).astype(np.float16)
    idx, val = oracle_mod.lut_argmax(p, x)
    ref = _lut_library(p, x)
    assert np.array_equal(idx, np.argmax(ref, axis=1))
    assert np.allclose(val, ref.max(axis=1), rtol=1e-12)


# ---- 2x16 vector LUT (model card, Release 0.2 format table, previous packages' MLP format)

def test_vq2_weight_hand_example(oracle_mod):
    """16 rows (two codebook groups), 2 columns, worked by hand: row r takes component r % 2 of
    centroid codes[r // 2][j] from group r // 8, times sc[r]."""
    cb = np.zeros((2, 16, 2), np.float16)
    cb[0, 3] = (0.5, -1.0)
    cb[0, 15] = (2.0, 0.25)
    cb[1, 3] = (-4.0, 8.0)
    cb[1, 0] = (1.5, -0.5)
    sc = np.ones(16, np.float16)
    sc[1], sc[9], sc[14] = 2.0, 0.5, -1.0
    codes = np.zeros((8, 2), np.uint8)
    codes[0] = (3, 15)   # rows 0, 1 (group 0)
    codes[4] = (3, 0)    # rows 8, 9 (group 1)
    codes[7] = (0, 3)    # rows 14, 15 (group 1)
    W = oracle_mod.vq2_weight(codes, cb, sc)
    assert W[0].tolist() == [0.5, 2.0]
    assert W[1].tolist() == [-2.0, 0.5]          # component 1, scale 2
    assert W[8].tolist() == [-4.0, 1.5]
    assert W[9].tolist() == [4.0, -0.25]         # component 1, scale 0.5
    assert W[14].tolist() == [-1.5, 4.0]         # component 0, scale -1
    assert W[15].tolist() == [-0.5, 8.0]
    assert not W[2:8].any()                      # group 0, centroid 0 is zero
    assert W[10:14].tolist() == [[1.5, 1.5], [-0.5, -0.5]] * 2  # group 1, centroid 0
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.vq2_weight(np.full((8, 2), 16, np.uint8), cb, sc)


def test_vq2_is_vq3_with_a_padded_codebook(oracle_mod):
    """With its 16 centroids placed first in a 64-entry codebook, a 2x16 matrix is a three-bit
    matrix with codes below 16: the numpy decode equals the C oracle's VQ3 decode exactly."""
    m = synth.vq2_matrix(np.random.default_rng(5), 48, 37)
    cb64 = np.zeros((6, 64, 2), np.float16)
    cb64[:, :16] = m.cb
    assert np.array_equal(oracle_mod.vq2_weight(m.codes, m.cb, m.sc),
                          oracle_mod.vq3_weight(m.codes, cb64.view(np.uint16), m.sc.view(np.uint16)))


def test_vq2_matmul_brute_force(oracle_mod):
    m = synth.vq2_matrix(np.random.default_rng(6), 16, 5)
    x = np.random.default_rng(7).standard_normal((3, 5)).astype(np.float16)
    cb, sc, xv = m.cb.astype(np.float64), m.sc.astype(np.float64), x.astype(np.float64)
    want = np.zeros((3, 16))
    for t in range(3):
        for r in range(16):
            for j in range(5):
                want[t, r] += cb[r // 8, m.codes[r // 2, j], r % 2] * sc[r] * xv[t, j]
    np.testing.assert_allclose(oracle_mod.vq2_matmul(m.codes, m.cb, m.sc, x), want, rtol=1e-13, atol=1e-15)


def test_vq2_mlp_is_vq3_mlp_with_padded_codebooks(oracle_mod):
    """The 2x16 MLP oracle (numpy products over materialised 2x16 weights) against the C oracle's
    three-bit MLP (weights decoded on the fly, sums in index order) on the same layer with every
    16-entry codebook placed first in a 64-entry one: two independent implementations of the same
    definition, equal up to summation order."""
    L = synth.vq2_mlp_layer(128, 256, 3, seed=8, outliers=True)
    y2 = oracle_mod.vq2_mlp_forward(L)

    def pad(m):
        cb = np.zeros((m.N // 8, 64, 2), np.float16)
        cb[:, :16] = m.cb
        return synth.VQ3Matrix(m.codes, cb, m.sc)

    L3 = synth.MLPLayer(L.H, L.I, L.T, L.x, L.s, L.sign_h, L.sign_i, pad(L.gate), pad(L.up),
                        pad(L.down), L.had_block_h, L.had_block_i)
    y3 = oracle_mod.mlp_forward(L3)
    assert np.linalg.norm(y2 - y3) <= 1e-12 * np.linalg.norm(y3)
    # token independence (BLAS may order a one-row product's sums differently)
    y1 = oracle_mod.vq2_mlp_forward(L, tokens=[1])
    assert np.linalg.norm(y1 - y2[1:2]) <= 1e-13 * np.linalg.norm(y2[1:2])


def test_vq2_mlp_identity_weights_closed_form(oracle_mod):
    """2x16 codebooks can hold the identity (entries (1, 0), (0, 1), (0, 0)): y = R_I(silu(x~) x~)."""
    n = 64
    L = synth.vq2_mlp_layer(n, n, 2, seed=4)
    cb = np.zeros((n // 8, 16, 2), np.float16)
    cb[:, 1, 0] = 1
    cb[:, 2, 1] = 1
    codes = np.zeros((n // 2, n), np.uint8)
    for p in range(n // 2):
        codes[p, 2 * p], codes[p, 2 * p + 1] = 1, 2
    ident = synth.VQ2Matrix(codes, cb, np.ones(n, np.float16))
    L.gate = L.up = L.down = ident
    y = oracle_mod.vq2_mlp_forward(L)
    xt = _blockdiag_rotate_ref(L.x.astype(np.float64) * L.s.astype(np.float64), L.had_block_h,
                               L.sign_h)
    expect = _blockdiag_rotate_ref(xt * scipy.special.expit(xt) * xt, L.had_block_i, L.sign_i)
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-14)
