"""CPU tests of the C-ABI library's host half: symbol exports, packing and argument checks.

No compute call is made here (there is no GPU in this tier); the packed layout is checked bit by
bit against the layout the header documents, and every documented error code is provoked.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from bit_vector_lut_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vqmlp.h")


@pytest.fixture(scope="module")
def vq():
    from bit_vector_lut_amd import vqmlp

    vqmlp.lib()
    return vqmlp


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vqmlp_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(vq):
    names = _declared_symbols()
    assert len(names) >= 17
    for n in names:
        assert hasattr(vq.lib(), n), n


def test_abi_version(vq):
    assert vq.lib().vqmlp_abi_version() == 1


@pytest.mark.parametrize("N,K", [(32, 64), (64, 128), (704, 256), (256, 704), (96, 192)])
def test_pack_unpack_round_trip(vq, N, K):
    m = synth.vq3_matrix(np.random.default_rng(N + K), N, K)
    packed = vq.pack(*m.as_u16())
    assert packed.size == vq.packed_bytes(N, K)
    codes, cb, sc = vq.unpack(N, K, packed)
    assert np.array_equal(codes, m.codes)
    assert np.array_equal(cb.view(np.uint16), m.cb.view(np.uint16))
    assert np.array_equal(sc.view(np.uint16), m.sc.view(np.uint16))


def test_packed_size_is_three_bits_per_weight(vq):
    N, K = 17408, 5120
    n = vq.packed_bytes(N, K)
    codes = N * K * 3 // 8
    cb = N // 8 * 64 * 4
    sc = N * 2
    assert codes + cb + sc <= n <= codes + cb + sc + 4 * 256


def test_code_positions_follow_documented_layout(vq):
    """Place single distinct codes and find them where the header says they are."""
    N, K = 64, 128
    rng = np.random.default_rng(0)
    m = synth.vq3_matrix(rng, N, K)
    packed = vq.pack(*m.as_u16())
    hdr = np.frombuffer(packed[:96].tobytes(), np.uint32)
    assert hdr[0] == 0x50335156 and hdr[1] == 1 and hdr[2] == N and hdr[3] == K
    codes_off = int(np.frombuffer(packed[32:40].tobytes(), np.uint64)[0])
    KT = K // 64
    bits = np.unpackbits(packed[codes_off:], bitorder="little")
    for _ in range(200):
        p, j = rng.integers(0, N // 2), rng.integers(0, K)
        mt, pi = divmod(p, 16)
        kt, cc = divmod(j, 64)
        s, rem = divmod(cc, 16)
        kc, i = divmod(rem, 4)
        lane = 16 * kc + pi
        q = 4 * s + i
        start = ((mt * KT + kt) * 768 + 12 * lane) * 8 + 6 * q
        val = int(np.dot(bits[start:start + 6], 1 << np.arange(6)))
        assert val == m.codes[p, j]


def test_pack_rejects_bad_input(vq):
    m = synth.vq3_matrix(np.random.default_rng(1), 64, 64)
    bad = m.codes.copy()
    bad[3, 5] = 64
    with pytest.raises(vq.VqmlpError) as e:
        vq.pack(bad, m.cb, m.sc)
    assert e.value.status == vq.ERR_INVALID_ARG and "> 63" in str(e.value)
    for N, K in [(48, 64), (64, 96), (0, 64), (64, -64)]:
        with pytest.raises(vq.VqmlpError) as e:
            vq.packed_bytes(N, K)
        assert e.value.status == vq.ERR_INVALID_ARG
    L = vq.lib()
    n = vq.packed_bytes(64, 64)
    buf = np.zeros(n - 1, np.uint8)
    codes, cb, sc = m.as_u16()
    st = L.vqmlp_pack(64, 64, codes.ctypes.data, cb.ctypes.data, sc.ctypes.data,
                      buf.ctypes.data, buf.size)
    assert st == vq.ERR_INVALID_ARG and b"needs" in L.vqmlp_last_error()
    st = L.vqmlp_pack(64, 64, None, cb.ctypes.data, sc.ctypes.data, buf.ctypes.data, n)
    assert st == vq.ERR_INVALID_ARG


def test_unpack_rejects_corrupt_header(vq):
    m = synth.vq3_matrix(np.random.default_rng(2), 64, 64)
    packed = vq.pack(*m.as_u16())
    for off, val, msg in [(0, 0x11, "magic"), (4, 2, "layout version"), (8, 32, "shape"),
                          (24, 2, "kind")]:
        bad = packed.copy()
        bad[off] = val
        with pytest.raises(vq.VqmlpError) as e:
            vq.unpack(64, 64, bad)
        assert e.value.status == vq.ERR_INVALID_ARG and msg in str(e.value), str(e.value)


@pytest.mark.parametrize("bits", [2, 4])
def test_lut_pack_round_trip(vq, bits):
    p = synth.lut_projection(np.random.default_rng(bits), bits, 128, 192, 0, 0)
    packed = vq.lut_pack(bits, p.codes, p.lut, p.sc)
    assert packed.size == vq.lut_packed_bytes(bits, 128, 192)
    codes, lut, sc = vq.lut_unpack(bits, 128, 192, packed)
    assert np.array_equal(codes, p.codes)
    assert np.array_equal(lut.view(np.uint16), p.lut.view(np.uint16))
    assert np.array_equal(sc.view(np.uint16), p.sc.view(np.uint16))
    bad = p.codes.copy()
    bad[0, 0] = 1 << bits
    with pytest.raises(vq.VqmlpError):
        vq.lut_pack(bits, bad, p.lut, p.sc)


def test_null_arguments_are_rejected_without_device(vq):
    L = vq.lib()
    plan = C.c_void_p()
    assert L.vqmlp_create(None, C.byref(plan)) == vq.ERR_INVALID_ARG
    assert L.vqmlp_forward(None, 1, None, None, None, 0, None) == vq.ERR_INVALID_ARG
    n = C.c_size_t()
    assert L.vqmlp_workspace_bytes(None, 1, C.byref(n)) == vq.ERR_INVALID_ARG
    assert L.vqmlp_rotate(1, 96, 64, None, None, None, None, None) == vq.ERR_INVALID_ARG
    assert L.vqmlp_rotate(1, 128, 3, None, None, None, None, None) == vq.ERR_INVALID_ARG
    assert L.vqmlp_dequant(48, 64, None, None, None) == vq.ERR_INVALID_ARG
    lf = L.vqmlp_lut_forward
    assert lf(3, 64, 64, 1, None, None, None, 0, None, None, 0, None, None, None, 0,
              None) == vq.ERR_INVALID_ARG  # bits
    assert lf(2, 32, 64, 1, None, None, None, 0, None, None, 0, None, None, None, 0,
              None) == vq.ERR_INVALID_ARG  # N % 64
    assert lf(2, 64, 64, 1, None, None, None, 300, None, None, 0, None, None, None, 0,
              None) == vq.ERR_INVALID_ARG  # rank
    assert lf(2, 64, 192, 1, None, None, None, 0, None, None, 128, None, None, None, 0,
              None) == vq.ERR_INVALID_ARG  # block does not divide K
    assert lf(2, 64, 64, 0, None, None, None, 0, None, None, 0, None, None, None, 0,
              None) == vq.OK  # empty batch
    assert lf(2, 64, 64, 2, None, None, None, 0, None, None, 0, None, None, None, 0,
              None) == vq.ERR_INVALID_ARG  # null buffers
    assert L.vqmlp_lut_workspace_bytes(64, 64, 1, 257, C.byref(n)) == vq.ERR_INVALID_ARG
    lp = C.c_void_p()
    lc = L.vqmlp_lut_create
    assert lc(3, 64, 64, None, None, None, 0, None, None, 0, C.byref(lp)) == vq.ERR_INVALID_ARG
    assert lc(2, 64, 192, None, None, None, 0, None, None, 128, C.byref(lp)) == vq.ERR_INVALID_ARG
    assert lc(2, 64, 64, None, None, None, 0, None, None, 0, C.byref(lp)) == vq.ERR_INVALID_ARG
    assert lc(2, 64, 64, None, None, None, 0, None, None, 0, None) == vq.ERR_INVALID_ARG
    assert not lp.value  # no plan on failure
    assert L.vqmlp_lut_plan_forward(None, 1, None, None, None, 0, None) == vq.ERR_INVALID_ARG
    assert L.vqmlp_last_error() != b""
    assert L.vqmlp_lut_destroy(None) == vq.OK


def test_lut_argmax_rejects_null_plan(vq):
    L = vq.lib()
    assert L.vqmlp_lut_plan_argmax(None, 1, None, None, None, None, 0, None) == vq.ERR_INVALID_ARG
    assert b"null plan" in L.vqmlp_last_error()


def test_vq2_pack_round_trip(vq):
    m = synth.vq2_matrix(np.random.default_rng(3), 64, 96)
    packed = vq.vq2_pack(m.codes, m.cb, m.sc)
    assert packed.size == vq.vq2_packed_bytes(64, 96) and packed.size % 256 == 0
    codes, cb, sc = vq.vq2_unpack(64, 96, packed)
    assert np.array_equal(codes, m.codes)
    assert np.array_equal(cb, m.cb.view(np.uint16))
    assert np.array_equal(sc, m.sc.view(np.uint16))


def test_vq2_pack_rejects_bad_codes_and_shapes(vq):
    m = synth.vq2_matrix(np.random.default_rng(4), 32, 32)
    codes = m.codes.copy()
    codes[3, 5] = 16
    with pytest.raises(vq.VqmlpError, match="code 16 > 15"):
        vq.vq2_pack(codes, m.cb, m.sc)
    with pytest.raises(vq.VqmlpError, match="multiples of 32"):
        vq.vq2_packed_bytes(40, 32)
    # a scalar-LUT buffer of the same shape is refused by its header kind
    lut = vq.lut_pack(2, np.zeros((64, 64), np.uint8), np.zeros((8, 4), np.float16),
                      np.ones(64, np.float16))
    lut = np.concatenate([lut, np.zeros(vq.vq2_packed_bytes(64, 64), np.uint8)])
    with pytest.raises(vq.VqmlpError, match="packed kind"):
        vq.vq2_unpack(64, 64, lut)
