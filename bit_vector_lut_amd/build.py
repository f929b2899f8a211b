"""Build the HIP library libvqmlp.so in-tree for gfx950 (hipcc cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libvqmlp.so")
SOURCES = ["vqmlp_host.cpp", "kernels.hip", "fused.hip", "tiled.hip", "vq3mm.hip", "lut8.hip",
           "vq2.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are kept out of the generated code: hipcc -O3 would otherwise form
# them from scalar float code by itself.
# The atomic optimizer is off: it turns a single-lane atomic whose result is used much later into
# a wave-wide reduction that needs the result at once, which stalls the code stream.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# Per-source flags.  The register-decode product is one wave per SIMD with long independent
# chains (cross-lane reads, matrix-core steps): the ILP-first scheduler batches its LDS reads and
# keeps the accumulators in place, where the default one serialises them to save registers.
# The fused T <= 8 kernel measured 1-2% faster per layer with the same scheduler (its product loop
# then keeps more lookups in flight ahead of the matrix-core steps).
SOURCE_FLAGS = {"vq3mm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
                "fused.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def build(verbose: bool = False) -> str:
    """Compile every source and link libvqmlp.so; always recompiles."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
