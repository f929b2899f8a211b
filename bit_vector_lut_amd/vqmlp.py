"""ctypes binding of libvqmlp.so (include/vqmlp.h).

Argument marshalling only: every step of the forward runs in the HIP kernels of the library.
PyTorch supplies device memory and the current HIP stream.  A missing library raises at import
of the first call; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvqmlp.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
PATH_AUTO, PATH_FUSED, PATH_TILED = 0, 1, 2


class VqmlpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("vqmlp status %d: %s" % (status, msg))
        self.status = status


class _Desc(C.Structure):
    _fields_ = [("H", C.c_int), ("I", C.c_int), ("had_block_h", C.c_int),
                ("had_block_i", C.c_int), ("t_max", C.c_int),
                ("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p),
                ("s_in", C.c_void_p), ("sign_h", C.c_void_p), ("sign_i", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libvqmlp.so is not built (run __graft_entry__.build() or "
                              "python bit_vector_lut_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        P, I, S = C.c_void_p, C.c_int, C.c_size_t
        L.vqmlp_abi_version.restype = I
        L.vqmlp_last_error.restype = C.c_char_p
        sigs = {
            "vqmlp_packed_bytes": [I, I, C.POINTER(S)],
            "vqmlp_pack": [I, I, P, P, P, P, S],
            "vqmlp_unpack": [I, I, P, S, P, P, P],
            "vqmlp_dequant": [I, I, P, P, P],
            "vqmlp_create": [C.POINTER(_Desc), C.POINTER(P)],
            "vqmlp_create_vq2": [C.POINTER(_Desc), C.POINTER(P)],
            "vqmlp_destroy": [P],
            "vqmlp_workspace_bytes": [P, I, C.POINTER(S)],
            "vqmlp_forward": [P, I, P, P, P, S, P],
            "vqmlp_forward_path": [P, I, P, P, P, S, I, P],
            "vqmlp_workspace_errors": [P, S, I, C.POINTER(C.c_uint32), P],
            "vqmlp_stream_read": [P, S, P, P],
            "vqmlp_forward_noalloc": [P, I, P, P, P],
            "vqmlp_rotate": [I, I, I, P, P, P, P, P],
            "vqmlp_lut_packed_bytes": [I, I, I, C.POINTER(S)],
            "vqmlp_lut_pack": [I, I, I, P, P, P, P, S],
            "vqmlp_lut_unpack": [I, I, I, P, S, P, P, P],
            "vqmlp_lut_workspace_bytes": [I, I, I, I, C.POINTER(S)],
            "vqmlp_lut_forward": [I, I, I, I, P, P, P, I, P, P, I, P, P, P, S, P],
            "vqmlp_lut_create": [I, I, I, P, P, P, I, P, P, I, C.POINTER(P)],
            "vqmlp_lut_destroy": [P],
            "vqmlp_lut_plan_forward": [P, I, P, P, P, S, P],
            "vqmlp_lut_plan_argmax": [P, I, P, P, P, P, S, P],
            "vqmlp_vq2_packed_bytes": [I, I, C.POINTER(S)],
            "vqmlp_vq2_pack": [I, I, P, P, P, P, S],
            "vqmlp_vq2_unpack": [I, I, P, S, P, P, P],
            "vqmlp_vq2_create": [I, I, P, C.POINTER(P)],
            "vqmlp_vq2_destroy": [P],
            "vqmlp_vq2_plan_forward": [P, I, P, P, P],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = I
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise VqmlpError(status, lib().vqmlp_last_error().decode())


def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.uint16, copy=False)


def _dptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ host-side packing


def packed_bytes(N: int, K: int) -> int:
    n = C.c_size_t()
    _check(lib().vqmlp_packed_bytes(N, K, C.byref(n)))
    return n.value


def pack(codes, cb, sc) -> np.ndarray:
    """Pack one VQ3 matrix (codes [N/2,K] uint8, cb [N/8,64,2] f16, sc [N] f16) -> uint8."""
    codes = np.ascontiguousarray(codes, np.uint8)
    cb, sc = _u16(cb), _u16(sc)
    N, K = sc.shape[0], codes.shape[1]
    out = np.empty(packed_bytes(N, K), np.uint8)
    _check(lib().vqmlp_pack(N, K, _np_ptr(codes), _np_ptr(cb), _np_ptr(sc), _np_ptr(out),
                            out.size))
    return out


def unpack(N: int, K: int, packed):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.empty((N // 2, K), np.uint8)
    cb = np.empty((N // 8, 64, 2), np.uint16)
    sc = np.empty(N, np.uint16)
    _check(lib().vqmlp_unpack(N, K, _np_ptr(packed), packed.size, _np_ptr(codes), _np_ptr(cb),
                              _np_ptr(sc)))
    return codes, cb.view(np.float16), sc.view(np.float16)


def lut_packed_bytes(bits: int, N: int, K: int) -> int:
    n = C.c_size_t()
    _check(lib().vqmlp_lut_packed_bytes(bits, N, K, C.byref(n)))
    return n.value


def lut_pack(bits: int, codes, lut, sc) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    lut, sc = _u16(lut), _u16(sc)
    N, K = codes.shape
    out = np.empty(lut_packed_bytes(bits, N, K), np.uint8)
    _check(lib().vqmlp_lut_pack(bits, N, K, _np_ptr(codes), _np_ptr(lut), _np_ptr(sc),
                                _np_ptr(out), out.size))
    return out


def lut_unpack(bits: int, N: int, K: int, packed):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.empty((N, K), np.uint8)
    lut = np.empty((N // 8, 1 << bits), np.uint16)
    sc = np.empty(N, np.uint16)
    _check(lib().vqmlp_lut_unpack(bits, N, K, _np_ptr(packed), packed.size, _np_ptr(codes),
                                  _np_ptr(lut), _np_ptr(sc)))
    return codes, lut.view(np.float16), sc.view(np.float16)


# ------------------------------------------------------------------ device side (torch)


def vq2_packed_bytes(N: int, K: int) -> int:
    n = C.c_size_t()
    _check(lib().vqmlp_vq2_packed_bytes(N, K, C.byref(n)))
    return n.value


def vq2_pack(codes, cb, sc) -> np.ndarray:
    """2x16 matrix: codes uint8 [N/2, K] (0..15), cb [N/8, 16, 2] and sc [N] binary16."""
    codes = np.ascontiguousarray(codes, np.uint8)
    cb, sc = _u16(cb), _u16(sc)
    N, K = sc.shape[0], codes.shape[1]
    out = np.empty(vq2_packed_bytes(N, K), np.uint8)
    _check(lib().vqmlp_vq2_pack(N, K, _np_ptr(codes), _np_ptr(cb), _np_ptr(sc), _np_ptr(out),
                                out.size))
    return out


def vq2_unpack(N: int, K: int, packed):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.empty((N // 2, K), np.uint8)
    cb = np.empty((N // 8, 16, 2), np.uint16)
    sc = np.empty(N, np.uint16)
    _check(lib().vqmlp_vq2_unpack(N, K, _np_ptr(packed), packed.size, _np_ptr(codes),
                                  _np_ptr(cb), _np_ptr(sc)))
    return codes, cb, sc


def to_device(a, device="cuda"):
    """numpy -> torch device tensor (float16 kept as its bits in int16)."""
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def workspace_errors(workspace, clear: bool = True, stream=None) -> int:
    """Error bits of the fused kernel's bounded waits in a forward workspace (0 = none); waits
    for the stream and, with clear, zeroes the word."""
    bits = C.c_uint32()
    _check(lib().vqmlp_workspace_errors(_dptr(workspace), workspace.numel(), int(clear),
                                        C.byref(bits), _stream(stream)))
    return bits.value


def stream_read(buf, sink, stream=None):
    """Measurement hook: one streaming read of the device tensor buf (bytes a multiple of 16)."""
    _check(lib().vqmlp_stream_read(_dptr(buf), buf.numel() * buf.element_size(), _dptr(sink),
                                   _stream(stream)))


def dequant(N: int, K: int, packed_dev, stream=None):
    import torch

    w = torch.empty((N, K), dtype=torch.float32, device=packed_dev.device)
    _check(lib().vqmlp_dequant(N, K, _dptr(packed_dev), _dptr(w), _stream(stream)))
    return w


def rotate(x_dev, b: int, s_dev=None, sign_dev=None, stream=None):
    """FP32 rotation test hook; x_dev int16 (binary16 bits) or float16 [T, n]."""
    import torch

    T, n = x_dev.shape
    out = torch.empty((T, n), dtype=torch.float32, device=x_dev.device)
    _check(lib().vqmlp_rotate(T, n, b, _dptr(x_dev), _dptr(s_dev), _dptr(sign_dev), _dptr(out),
                              _stream(stream)))
    return out


class MLP:
    """Device-resident packed weights of one MLP layer plus its plan."""

    def __init__(self, H, I, gate, up, down, s, sign_h=None, sign_i=None, had_block_h=0,
                 had_block_i=0, t_max=512, vq2=False):
        """vq2: the three matrices are packed 2x16 buffers (vq2_pack), else three-bit (pack)."""
        self.H, self.I, self.t_max = H, I, t_max
        self._keep = (gate, up, down, s, sign_h, sign_i)  # the plan does not own these
        d = _Desc(H, I, had_block_h, had_block_i, t_max, gate.data_ptr(), up.data_ptr(),
                  down.data_ptr(), s.data_ptr(),
                  sign_h.data_ptr() if sign_h is not None else None,
                  sign_i.data_ptr() if sign_i is not None else None)
        self._plan = C.c_void_p()
        create = lib().vqmlp_create_vq2 if vq2 else lib().vqmlp_create
        _check(create(C.byref(d), C.byref(self._plan)))
        self.device = gate.device

    @classmethod
    def from_layer(cls, layer, device="cuda", t_max=None):
        """Pack a ``synth.MLPLayer`` on the host and upload it."""
        packs = [to_device(pack(*m.as_u16()), device) for m in (layer.gate, layer.up, layer.down)]
        return cls(layer.H, layer.I, *packs, to_device(layer.s, device),
                   to_device(layer.sign_h, device), to_device(layer.sign_i, device),
                   layer.had_block_h, layer.had_block_i,
                   t_max if t_max is not None else max(layer.T, 8))

    @classmethod
    def from_vq2_layer(cls, layer, device="cuda", t_max=None):
        """Pack a ``synth.vq2_mlp_layer`` (2x16 matrices) on the host and upload it."""
        packs = [to_device(vq2_pack(*m.as_u16()), device) for m in (layer.gate, layer.up, layer.down)]
        return cls(layer.H, layer.I, *packs, to_device(layer.s, device),
                   to_device(layer.sign_h, device), to_device(layer.sign_i, device),
                   layer.had_block_h, layer.had_block_i,
                   t_max if t_max is not None else max(layer.T, 8), vq2=True)

    def workspace_bytes(self, T: int) -> int:
        n = C.c_size_t()
        _check(lib().vqmlp_workspace_bytes(self._plan, T, C.byref(n)))
        return n.value

    def workspace(self, T=None):
        import torch

        return torch.zeros(self.workspace_bytes(self.t_max if T is None else T),
                           dtype=torch.uint8, device=self.device)

    def forward(self, x, y=None, workspace=None, path=PATH_AUTO, stream=None):
        """x: [T, H] int16 (binary16 bits) or float16 device tensor -> y (same dtype)."""
        import torch

        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        if workspace is None:
            workspace = self.workspace(T)
        _check(lib().vqmlp_forward_path(self._plan, T, _dptr(x), _dptr(y), _dptr(workspace),
                                        workspace.numel(), path, _stream(stream)))
        return y

    def forward_noalloc(self, x, y=None, stream=None):
        """The forward with the library's fixed per-GPU scratch array as its workspace."""
        import torch

        if y is None:
            y = torch.empty_like(x)
        _check(lib().vqmlp_forward_noalloc(self._plan, x.shape[0], _dptr(x), _dptr(y),
                                           _stream(stream)))
        return y

    def __del__(self):
        if getattr(self, "_plan", None) and _lib is not None:
            _lib.vqmlp_destroy(self._plan)
            self._plan = None


class LUTProjection:
    """Device-resident scalar-LUT projection (2- or 4-bit codes, group-8 tables, optional
    rank-r factors) with its input scale, sign and Hadamard block."""

    def __init__(self, bits, N, K, packed, U=None, V=None, s=None, sign=None, had_block=1024):
        self.bits, self.N, self.K = bits, N, K
        self.r = 0 if U is None else U.shape[1]
        self.had_block = had_block
        self.packed, self.U, self.V, self.s, self.sign = packed, U, V, s, sign
        self.device = packed.device
        self._plan = C.c_void_p()
        _check(lib().vqmlp_lut_create(bits, N, K, _dptr(packed), _dptr(U), _dptr(V), self.r,
                                      _dptr(s), _dptr(sign), had_block, C.byref(self._plan)))

    @classmethod
    def from_proj(cls, proj, device="cuda"):
        """Pack a ``synth.LUTProjection`` on the host and upload it."""
        packed = to_device(lut_pack(proj.bits, proj.codes, proj.lut, proj.sc), device)
        up = lambda a: None if a is None else to_device(a, device)  # noqa: E731
        return cls(proj.bits, proj.N, proj.K, packed, up(proj.U), up(proj.V), up(proj.s),
                   up(proj.sign), proj.had_block)

    def workspace_bytes(self, T: int) -> int:
        n = C.c_size_t()
        _check(lib().vqmlp_lut_workspace_bytes(self.N, self.K, T, self.r, C.byref(n)))
        return n.value

    def workspace(self, T: int):
        import torch

        return torch.zeros(self.workspace_bytes(T), dtype=torch.uint8, device=self.device)

    def forward(self, x, y=None, workspace=None, stream=None):
        """x: [T, K] int16 (binary16 bits) or float16 device tensor -> y [T, N] (same dtype)."""
        import torch

        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.N), dtype=x.dtype, device=x.device)
        if workspace is None:
            workspace = self.workspace(T)
        _check(lib().vqmlp_lut_plan_forward(self._plan, T, _dptr(x), _dptr(y), _dptr(workspace),
                                            workspace.numel(), _stream(stream)))
        return y

    def argmax(self, x, workspace=None, stream=None):
        """Greedy argmax head: x [T, K] float16 device tensor (T <= 8) -> (index int32 [T],
        value float32 [T]): per token the lowest row of the largest logit, and that logit."""
        import torch

        T = x.shape[0]
        index = torch.empty(T, dtype=torch.int32, device=x.device)
        value = torch.empty(T, dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = self.workspace(T)
        _check(lib().vqmlp_lut_plan_argmax(self._plan, T, _dptr(x), _dptr(index), _dptr(value),
                                           _dptr(workspace), workspace.numel(), _stream(stream)))
        return index, value

    def forward_stateless(self, x, y=None, workspace=None, stream=None):
        """The same through vqmlp_lut_forward (validates the packed buffer on every call)."""
        import torch

        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.N), dtype=x.dtype, device=x.device)
        if workspace is None:
            workspace = self.workspace(T)
        _check(lib().vqmlp_lut_forward(self.bits, self.N, self.K, T, _dptr(self.packed),
                                       _dptr(self.U), _dptr(self.V), self.r, _dptr(self.s),
                                       _dptr(self.sign), self.had_block, _dptr(x), _dptr(y),
                                       _dptr(workspace), workspace.numel(), _stream(stream)))
        return y

    def __del__(self):
        if getattr(self, "_plan", None) and _lib is not None:
            _lib.vqmlp_lut_destroy(self._plan)
            self._plan = None


class VQ2Projection:
    """Device-resident 2x16 vector-LUT projection for T <= 8 tokens (x used as given)."""

    def __init__(self, N, K, packed):
        self.N, self.K, self.packed = N, K, packed
        self._plan = C.c_void_p()
        _check(lib().vqmlp_vq2_create(N, K, _dptr(packed), C.byref(self._plan)))

    @classmethod
    def from_matrix(cls, m, device="cuda"):
        """Pack a ``synth.VQ2Matrix`` on the host and upload it."""
        return cls(m.N, m.K, to_device(vq2_pack(m.codes, m.cb, m.sc), device))

    def forward(self, x, y=None, stream=None):
        """x: [T, K] binary16 device tensor (T <= 8) -> y [T, N] (same dtype)."""
        import torch

        if y is None:
            y = torch.empty((x.shape[0], self.N), dtype=x.dtype, device=x.device)
        _check(lib().vqmlp_vq2_plan_forward(self._plan, x.shape[0], _dptr(x), _dptr(y),
                                            _stream(stream)))
        return y

    def __del__(self):
        if getattr(self, "_plan", None) and _lib is not None:
            _lib.vqmlp_vq2_destroy(self._plan)
            self._plan = None

