"""ctypes wrapper of the FP64 CPU oracle (vqmlp_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU-baseline
leg, never by the HIP library or its binding.  Arguments are the unpacked arrays drawn by
``bit_vector_lut_amd.synth`` (plain numpy), so nothing here depends on the GPU path.

The arithmetic lives in vqmlp_oracle.c, whose header gives the definitions and the passages of
the pages they follow, except the 2x16 vector-LUT decode (``vq2_weight``, plain numpy; its
docstring cites its passage) and the argmax over ``lut_forward``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "vqmlp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP over output rows)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P, I, D = C.c_void_p, C.c_int, C.c_double
        L.orc_f16_to_f64.restype = D
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f16_array.argtypes = [C.c_size_t, P, P]
        L.orc_hadamard_entry.argtypes = [I, I]
        L.orc_hadamard.argtypes = [I, P]
        L.orc_rotate.argtypes = [I, I, I, P, P, P]
        L.orc_silu_1.restype = D
        L.orc_silu_1.argtypes = [D]
        L.orc_silu.argtypes = [C.c_size_t, P, P]
        L.orc_vq3_weight.argtypes = [I, I, P, P, P, P]
        L.orc_vq3_matmul.argtypes = [I, I, I, P, P, P, P, P]
        L.orc_mlp_forward.argtypes = [I] * 5 + [P] * 4 + [P] * 9 + [P] * 6
        L.orc_lut_weight.argtypes = [I, I, I, P, P, P, P]
        L.orc_lut_forward.argtypes = [I] * 6 + [P] * 3 + [P] * 5 + [P, P]
        L.orc_num_threads.restype = I
        L.orc_set_num_threads.argtypes = [I]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _u16(a):
    """float16 (or its raw bits) as contiguous uint16."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16, got %s" % a.dtype)
    return a


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc:
        raise OracleError("%s: invalid arguments" % what)


def f16_to_f64(h) -> np.ndarray:
    h = _u16(np.asarray(h))
    out = np.empty(h.shape, np.float64)
    lib().orc_f16_array(h.size, _p(h), _p(out))
    return out


def hadamard(b: int) -> np.ndarray:
    out = np.empty((b, b), np.int8)
    lib().orc_hadamard(b, _p(out))
    return out


def rotate(u, b: int, sign=None) -> np.ndarray:
    """Block Hadamard rotation of the rows of u (float64 [T, n]); sign (+-1 [n]) applied first."""
    u = np.ascontiguousarray(np.atleast_2d(u), np.float64)
    out = np.empty_like(u)
    _check(lib().orc_rotate(u.shape[0], u.shape[1], b, _p(u), _p(_c(sign, np.int8)), _p(out)),
           "rotate")
    return out


def silu(g) -> np.ndarray:
    g = np.ascontiguousarray(g, np.float64)
    out = np.empty_like(g)
    lib().orc_silu(g.size, _p(g), _p(out))
    return out


def vq3_weight(codes, cb, sc) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    cb, sc = _u16(cb), _u16(sc)
    N, K = sc.shape[0], codes.shape[1]
    W = np.empty((N, K), np.float64)
    _check(lib().orc_vq3_weight(N, K, _p(codes), _p(cb), _p(sc), _p(W)), "vq3_weight")
    return W


def vq3_matmul(codes, cb, sc, xin) -> np.ndarray:
    """out[t][r] = sum_j W[r][j] xin[t][j] with W decoded on the fly."""
    codes = np.ascontiguousarray(codes, np.uint8)
    cb, sc = _u16(cb), _u16(sc)
    xin = np.ascontiguousarray(np.atleast_2d(xin), np.float64)
    N, K = sc.shape[0], codes.shape[1]
    out = np.empty((xin.shape[0], N), np.float64)
    _check(lib().orc_vq3_matmul(xin.shape[0], N, K, _p(codes), _p(cb), _p(sc), _p(xin), _p(out)),
           "vq3_matmul")
    return out


def mlp_forward(layer, tokens=None, intermediates: bool = False):
    """FP64 forward of a ``synth.MLPLayer``; ``tokens`` selects rows of x (each token is
    independent).  Returns y [T', H] or, with intermediates, a dict with xt, g, v, a, at, y."""
    x = layer.x if tokens is None else layer.x[np.asarray(tokens)]
    x = _u16(x)
    T, H, I = x.shape[0], layer.H, layer.I
    y = np.empty((T, H), np.float64)
    inter = {}
    if intermediates:
        inter = {"xt": np.empty((T, H)), "g": np.empty((T, I)), "v": np.empty((T, I)),
                 "a": np.empty((T, I)), "at": np.empty((T, I))}
    mats = []
    for m in (layer.gate, layer.up, layer.down):
        mats += [np.ascontiguousarray(m.codes, np.uint8), _u16(m.cb), _u16(m.sc)]
    rc = lib().orc_mlp_forward(
        T, H, I, layer.had_block_h, layer.had_block_i, _p(x), _p(_u16(layer.s)),
        _p(_c(layer.sign_h, np.int8)), _p(_c(layer.sign_i, np.int8)),
        *[_p(a) for a in mats], _p(y),
        *[_p(inter.get(k)) for k in ("xt", "g", "v", "a", "at")])
    _check(rc, "mlp_forward")
    if intermediates:
        inter["y"] = y
        return inter
    return y


def lut_weight(bits, codes, lut, sc) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    lut, sc = _u16(lut), _u16(sc)
    N, K = codes.shape
    W = np.empty((N, K), np.float64)
    _check(lib().orc_lut_weight(bits, N, K, _p(codes), _p(lut), _p(sc), _p(W)), "lut_weight")
    return W


def lut_forward(proj, x, tokens=None, with_xt: bool = False):
    """FP64 forward of a ``synth.LUTProjection`` on x (float16 [T, K])."""
    x = x if tokens is None else x[np.asarray(tokens)]
    x = _u16(x)
    T, K = x.shape
    N = proj.N
    y = np.empty((T, N), np.float64)
    xt = np.empty((T, K), np.float64) if with_xt else None
    rank = proj.rank
    rc = lib().orc_lut_forward(
        proj.bits, N, K, T, proj.had_block, rank, _p(x), _p(_u16(proj.s)),
        _p(_c(proj.sign, np.int8)), _p(np.ascontiguousarray(proj.codes, np.uint8)),
        _p(_u16(proj.lut)), _p(_u16(proj.sc)), _p(_u16(proj.U)), _p(_u16(proj.V)), _p(y), _p(xt))
    _check(rc, "lut_forward")
    return (y, xt) if with_xt else y


def lut_argmax(proj, x, tokens=None):
    """Greedy next token of a scalar-LUT output head: per row of x, the index of the largest FP64
    logit of ``lut_forward`` (the lowest index among equal logits) and that logit.  In-model argmax
    ("ANEMLL ANE LLM conversion pipeline", section "Facts", in-model argmax item: the head returns
    an index and its value instead of the vocabulary's logits; the four-bit LUT head of the model
    card's format table)."""
    y = lut_forward(proj, x, tokens)
    idx = np.argmax(y, axis=1)  # first occurrence of the maximum
    return idx.astype(np.int64), y[np.arange(y.shape[0]), idx]


def vq2_weight(codes, cb, sc) -> np.ndarray:
    """Decoded 2x16 matrix in FP64: W[r][j] = cb[r // 8][codes[r // 2][j]][r % 2] * sc[r].

    The two-bit vector lookup table "2x16" of the MLP in the previous packages (model card
    "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP, token-mixer
    rotations, distilled weights", format table, "Previous packages" column): 16 two-component
    centroids, one four-bit index per pair of output channels, per-channel scales.  The vector
    axis, component order, group of 8 output rows per codebook and scale placement are the
    readings of the three-bit 2x64 form (vqmlp_oracle.c header) with 16 entries instead of 64.
    Written in numpy on its own: one row at a time, the centroid component times the scale."""
    codes = np.asarray(codes)
    if codes.size and int(codes.max()) > 15:
        raise OracleError("vq2_weight: code above 15")
    cbv = f16_to_f64(cb)
    scv = f16_to_f64(sc)
    N, K = scv.shape[0], codes.shape[1]
    if codes.shape[0] * 2 != N or cbv.shape != (N // 8, 16, 2) or N % 8:
        raise OracleError("vq2_weight: inconsistent shapes")
    W = np.empty((N, K), np.float64)
    for r in range(N):
        W[r] = cbv[r // 8][codes[r // 2].astype(np.int64), r % 2] * scv[r]
    return W


def vq2_matmul(codes, cb, sc, xin) -> np.ndarray:
    """out[t][r] = sum_j W[r][j] xin[t][j] for the 2x16 matrix (FP64; the operand is used as
    given: any input scale or rotation is the caller's)."""
    W = vq2_weight(codes, cb, sc)
    x = np.asarray(np.atleast_2d(xin))
    x = f16_to_f64(x) if x.dtype in (np.float16, np.uint16) else x.astype(np.float64)
    return x @ W.T


def vq2_mlp_forward(layer, tokens=None):
    """FP64 forward of an MLP layer whose three matrices are 2x16 vector LUTs (the previous
    packages' MLP format: model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2:
    three-bit MLP, token-mixer rotations, distilled weights", format table, "Previous packages"
    column).  The same steps as ``mlp_forward`` (that card's rotation and activation bullets):
    x~ = R_H(x . s), a = silu(W_gate x~) . (W_up x~) . sign_I rotated by R_I, y = W_down a~,
    composed from ``rotate``, ``silu`` and ``vq2_matmul``; each step is one of the oracle's
    pinned functions."""
    x = layer.x if tokens is None else layer.x[np.asarray(tokens)]
    u = f16_to_f64(x) * f16_to_f64(layer.s)[None, :]
    xt = rotate(u, layer.had_block_h, layer.sign_h)
    g = vq2_matmul(layer.gate.codes, layer.gate.cb, layer.gate.sc, xt)
    v = vq2_matmul(layer.up.codes, layer.up.cb, layer.up.sc, xt)
    a = silu(g) * v
    at = rotate(a, layer.had_block_i, layer.sign_i)
    return vq2_matmul(layer.down.codes, layer.down.cb, layer.down.sc, at)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (for timing it on one core)."""
    lib().orc_set_num_threads(int(n))


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
