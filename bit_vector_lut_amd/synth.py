"""Seeded synthetic inputs for the VQ3 quantized-MLP forward and the scalar-LUT projections.

This module only draws random numbers and rounds them to the storage types; it holds none of
the method's arithmetic (no decode, rotation, activation or product).  Both the FP64 oracle and
the HIP library consume exactly these arrays, so a layer is fully defined by its seed.

Every array is drawn from one ``numpy.random.Generator`` (PCG64) in a fixed order:

  1. x ~ N(0, 1), shape [T, H]; optionally round(0.01*H) outlier channels, drawn without
     replacement, are multiplied by 20 in every row; then rounded to float16 (nearest even);
  2. s ~ LogNormal(0, 0.3), shape [H] -> float16      (per-channel input scale);
  3. d_H = 2*integers(0, 2, H) - 1, d_I likewise [I]  (signs of the two rotations);
  4. for gate (N=I, K=H), up (N=I, K=H), down (N=H, K=I), in that order:
       codes = integers(0, 64, (N/2, K), uint8)        one 6-bit index per output-row pair;
       cb    = N(0, 0.02), shape (N/8, 64, 2) -> float16  64 two-component centroids per 8 rows;
       sc    = U(0.5, 1.5), shape (N,) -> float16     one scale per output row.

The weight format follows the model card "anemll/anemll-forge-qwen3.8-27B", section
"Release 0.2: three-bit MLP, token-mixer rotations, distilled weights" (format table and the
bullet on three bits per MLP weight): a 2x64 vector lookup table with one six-bit index per pair
of output channels and per-channel scales.  The distributions are those of the synthetic
workloads this library is measured on; there are no trained weights here.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16 = np.float16


@dataclass
class VQ3Matrix:
    """One VQ3 matrix W[N, K] in its unpacked form."""

    codes: np.ndarray  # uint8 [N/2, K], values 0..63; row p covers output rows 2p and 2p+1
    cb: np.ndarray  # float16 [N/8, 64, 2]; [g, c, 0] -> row 8g+2q, [g, c, 1] -> row 8g+2q+1
    sc: np.ndarray  # float16 [N]

    @property
    def N(self) -> int:
        return self.sc.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[1]

    def as_u16(self):
        """(codes, codebook bits, scale bits) as the C ABI takes them."""
        return (
            np.ascontiguousarray(self.codes),
            np.ascontiguousarray(self.cb).view(np.uint16),
            np.ascontiguousarray(self.sc).view(np.uint16),
        )


@dataclass
class MLPLayer:
    H: int
    I: int
    T: int
    x: np.ndarray  # float16 [T, H]
    s: np.ndarray  # float16 [H]
    sign_h: np.ndarray  # int8 [H], +-1
    sign_i: np.ndarray  # int8 [I], +-1
    gate: VQ3Matrix
    up: VQ3Matrix
    down: VQ3Matrix
    had_block_h: int = 128
    had_block_i: int = 128
    meta: dict = field(default_factory=dict)


def default_block(n: int, cap: int = 128) -> int:
    """Largest power of two <= cap that divides n (128 for 256/5120/17408, 64 for 704)."""
    b = 1
    while b * 2 <= cap and n % (b * 2) == 0:
        b *= 2
    return b


def _rng(seed) -> np.random.Generator:
    if isinstance(seed, np.random.Generator):
        return seed
    return np.random.default_rng(seed)


def vq3_matrix(rng: np.random.Generator, N: int, K: int) -> VQ3Matrix:
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    codes = rng.integers(0, 64, size=(N // 2, K), dtype=np.uint8)
    cb = rng.normal(0.0, 0.02, size=(N // 8, 64, 2)).astype(F16)
    sc = rng.uniform(0.5, 1.5, size=N).astype(F16)
    return VQ3Matrix(codes, cb, sc)


class VQ2Matrix(VQ3Matrix):
    """One 2x16 matrix W[N, K]: codes uint8 [N/2, K] with values 0..15, cb float16 [N/8, 16, 2]
    (same component and group conventions as VQ3Matrix), sc float16 [N]."""


def vq2_matrix(rng: np.random.Generator, N: int, K: int) -> VQ2Matrix:
    """Draw order: codes, codebook, scales (the distributions of vq3_matrix)."""
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    codes = rng.integers(0, 16, size=(N // 2, K), dtype=np.uint8)
    cb = rng.normal(0.0, 0.02, size=(N // 8, 16, 2)).astype(F16)
    sc = rng.uniform(0.5, 1.5, size=N).astype(F16)
    return VQ2Matrix(codes, cb, sc)


def signs(rng: np.random.Generator, n: int) -> np.ndarray:
    return (2 * rng.integers(0, 2, size=n) - 1).astype(np.int8)


def activations(rng: np.random.Generator, T: int, H: int, outliers: bool) -> np.ndarray:
    x = rng.standard_normal((T, H))
    if outliers:
        n_out = int(round(0.01 * H))
        idx = rng.choice(H, size=n_out, replace=False)
        x[:, idx] *= 20.0
    return x.astype(F16)


def mlp_layer(H: int, I: int, T: int, seed=0, outliers: bool = False,
              had_block_h: int | None = None, had_block_i: int | None = None) -> MLPLayer:
    """Draw one MLP layer (activations, input scale, signs, three VQ3 matrices)."""
    rng = _rng(seed)
    x = activations(rng, T, H, outliers)
    s = rng.lognormal(0.0, 0.3, size=H).astype(F16)
    sign_h = signs(rng, H)
    sign_i = signs(rng, I)
    gate = vq3_matrix(rng, I, H)
    up = vq3_matrix(rng, I, H)
    down = vq3_matrix(rng, H, I)
    return MLPLayer(H, I, T, x, s, sign_h, sign_i, gate, up, down,
                    had_block_h or default_block(H), had_block_i or default_block(I),
                    meta={"outliers": outliers})


def vq2_mlp_layer(H: int, I: int, T: int, seed=0, outliers: bool = False,
                  had_block_h: int | None = None, had_block_i: int | None = None) -> MLPLayer:
    """One MLP layer in the 2x16 format: the draw order of mlp_layer with vq2_matrix in place of
    vq3_matrix (codes 0..15, 16 centroids per 8 rows)."""
    rng = _rng(seed)
    x = activations(rng, T, H, outliers)
    s = rng.lognormal(0.0, 0.3, size=H).astype(F16)
    sign_h = signs(rng, H)
    sign_i = signs(rng, I)
    gate = vq2_matrix(rng, I, H)
    up = vq2_matrix(rng, I, H)
    down = vq2_matrix(rng, H, I)
    return MLPLayer(H, I, T, x, s, sign_h, sign_i, gate, up, down,
                    had_block_h or default_block(H), had_block_i or default_block(I),
                    meta={"outliers": outliers, "format": "2x16"})


# ---------------------------------------------------------------------------------------------
# Scalar-LUT projection (token-mixer format): one table of 2**bits float16 entries per 8 output
# rows, a float16 scale per output row and rank-r float16 factors U[N, r], V[r, K].  The input is
# scaled per channel and rotated by 1024-wide seeded Hadamard blocks before the product.
# ---------------------------------------------------------------------------------------------


@dataclass
class LUTProjection:
    bits: int
    codes: np.ndarray  # uint8 [N, K], values < 2**bits
    lut: np.ndarray  # float16 [N/8, 2**bits]
    sc: np.ndarray  # float16 [N]
    U: np.ndarray | None  # float16 [N, r]
    V: np.ndarray | None  # float16 [r, K]
    s: np.ndarray | None  # float16 [K] input scale
    sign: np.ndarray | None  # int8 [K]
    had_block: int

    @property
    def N(self) -> int:
        return self.sc.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[1]

    @property
    def rank(self) -> int:
        return 0 if self.U is None else self.U.shape[1]


def lut_projection(rng: np.random.Generator, bits: int, N: int, K: int, rank: int = 64,
                   had_block: int = 1024) -> LUTProjection:
    """Draw order: codes, lut, sc, U, V, s, sign."""
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    lut = rng.normal(0.0, 0.02, size=(N // 8, 1 << bits)).astype(F16)
    sc = rng.uniform(0.5, 1.5, size=N).astype(F16)
    U = V = None
    if rank:
        U = rng.normal(0.0, 0.01, size=(N, rank)).astype(F16)
        V = rng.normal(0.0, 0.01, size=(rank, K)).astype(F16)
    s = rng.lognormal(0.0, 0.3, size=K).astype(F16)
    sign = signs(rng, K)
    return LUTProjection(bits, codes, lut, sc, U, V, s, sign, had_block)


# ---------------------------------------------------------------------------------------------
# The five measured workloads.
# ---------------------------------------------------------------------------------------------

H27, I27 = 5120, 17408  # 27B-like MLP shape


def tiny_layer() -> MLPLayer:
    """Tiny single MLP: H=256, I=704, T=1, seed 0 (rotation blocks 128 and 64)."""
    return mlp_layer(256, 704, 1, seed=0, outliers=False)


def layer27b_t8() -> MLPLayer:
    """One 27B-like MLP at T=8 (anchor + 7 drafts), 1% outlier channels x20, seed 0."""
    return mlp_layer(H27, I27, 8, seed=0, outliers=True)


def layer27b_t64() -> MLPLayer:
    """The same shape at T=64 (fixed-size prefill chunk), no outliers, seed 0."""
    return mlp_layer(H27, I27, 64, seed=0, outliers=False)


def stream_seeds(n_layers: int = 64):
    """Per-layer generators of the 64-layer T=8 stream."""
    return [np.random.default_rng(c) for c in np.random.SeedSequence(0).spawn(n_layers)]


def stream_layer(i: int, n_layers: int = 64) -> MLPLayer:
    child = np.random.SeedSequence(0).spawn(n_layers)[i]
    return mlp_layer(H27, I27, 8, seed=np.random.default_rng(child), outliers=True)


def prefill512():
    """T=512 prefill: one 27B-like MLP, then a 2-bit and a 4-bit 5120x5120 scalar-LUT projection
    with rank-64 factors, all from one generator (MLP first, then 2-bit, then 4-bit).  The
    projections take the MLP's input x."""
    rng = np.random.default_rng(0)
    layer = mlp_layer(H27, I27, 512, seed=rng, outliers=False)
    p2 = lut_projection(rng, 2, H27, H27, 64, 1024)
    p4 = lut_projection(rng, 4, H27, H27, 64, 1024)
    return layer, p2, p4
