"""CPU tier: the host half of the C ABI and the oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc / g++, host code only) and driven by small C programs
(tests/sanitize/): packing round trips, argument errors, and oracle forwards on small inputs.
The HIP objects of the library are linked unchanged (no GPU call is made)."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(not shutil.which("gcc"), reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "vqmlp_oracle.c"), "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not shutil.which("g++") or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not found")
def test_host_abi_under_sanitizers(tmp_path):
    build = os.path.join(ROOT, "bit_vector_lut_amd", "_build")
    from bit_vector_lut_amd.build import SOURCES

    objs = [os.path.join(build, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        from bit_vector_lut_amd import build as hipbuild

        hipbuild.build()
    host = str(tmp_path / "host_san.o")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_vector_lut_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    _run(["g++", "-std=c++17", *SAN, *inc, "-c",
          os.path.join(ROOT, "bit_vector_lut_amd", "csrc", "vqmlp_host.cpp"), "-o", host])
    drv = str(tmp_path / "driver.o")
    _run(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "sanitize", "host_abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "host_abi_driver")
    _run(["g++", *SAN, "-o", exe, drv, host, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV)
    assert "host ABI driver: ok" in r.stdout
