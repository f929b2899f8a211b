"""VQ3 quantized-MLP forward for AMD MI355X (gfx950).

``bit_vector_lut_amd.synth`` draws seeded inputs; ``bit_vector_lut_amd.vqmlp`` is the ctypes
binding of the HIP library (imported lazily so that input generation needs no GPU stack).
"""

__all__ = ["synth", "vqmlp"]


def __getattr__(name):
    if name in ("vqmlp", "synth"):
        import importlib

        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
