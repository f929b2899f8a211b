"""Per-item timeline of the fused T <= 8 kernel (profiling tool; the library itself is untouched).

A copy of the kernel sources is patched with `s_memrealtime` probes (100 MHz) that record, per
workgroup: the kernel start and end, the time of the item loop's first barrier in each iteration,
the item taken, and each wave's start and end of the products of each item.  The records go to a
second half of an oversized workspace (16 MiB; the forward uses the first 8 MiB).  The patched copy
is built into bit_vector_lut_amd/_build/timeline/ and driven over several distinct 27B-like layers
cycled through (so the weights come from HBM); the summary is printed as Markdown.

  python -m bit_vector_lut_amd.fused_timeline build            # CPU: patch and compile
  python -m bit_vector_lut_amd.fused_timeline run [--layers 4]  # GPU: run and summarise
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "_build", "timeline")
LIB = os.path.join(OUT, "libvqmlp_timeline.so")
REC_OFF = 8 << 20   # byte offset of the records in the workspace
REC_WORDS = 1024    # 64-bit words per workgroup
MAX_WG = 1024       # workgroups the record area holds (the kernel runs one per compute unit)


def _patch(src: str) -> str:
    def rep(s, old, new):
        assert s.count(old) == 1, "instrumentation point not found: %r" % old[:60]
        return s.replace(old, new)
    rt = "__builtin_amdgcn_s_memrealtime()"
    s = rep(src, "    const unsigned limit = a.spin_limit;\n",
            "    const unsigned limit = a.spin_limit;\n"
            "    uint64_t* TL = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ctl) + %du) + "
            "size_t(blockIdx.x) * %d;\n"
            "    if (tid == 0) TL[0] = %s;\n" % (REC_OFF, REC_WORDS, rt))
    s = rep(s, "        __syncthreads();  // (A) tables of cur and partials of prev are complete\n",
            "        __syncthreads();  // (A) tables of cur and partials of prev are complete\n"
            "        if (tid == 0 && j < 14) { TL[2 + j] = %s; TL[400 + j] = uint64_t(cur_u) + 1; }\n" % rt)
    s = rep(s, "        // (H) the products; the code ring",
            "        if (l == 0 && j < 8) TL[16 + 16 * w + 2 * j] = %s;\n"
            "        // (H) the products; the code ring" % rt)
    s = rep(s, "            // (I) next item's tables into the idle buffers",
            "            if (l == 0 && j < 8) TL[17 + 16 * w + 2 * j] = %s;\n"
            "            // (I) next item's tables into the idle buffers" % rt)
    s = rep(s, "    __syncthreads();\n    if (tid == 0) {\n        const uint32_t done",
            "    __syncthreads();\n    if (tid == 0) TL[1] = %s;\n    if (tid == 0) {\n"
            "        const uint32_t done" % rt)
    return s


def build() -> str:
    """Patch a copy of the sources and compile the instrumented library (no GPU needed)."""
    from bit_vector_lut_amd import build as hipbuild

    src_dir = os.path.join(OUT, "src")
    shutil.rmtree(OUT, ignore_errors=True)
    shutil.copytree(os.path.join(PKG, "csrc"), src_dir)
    p = os.path.join(src_dir, "fused.hip")
    with open(p) as fh:
        s = _patch(fh.read())
    with open(p, "w") as fh:
        fh.write(s)
    objs = []
    for src in hipbuild.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [hipbuild.HIPCC, *hipbuild.HIP_FLAGS, *hipbuild.SOURCE_FLAGS.get(src, []),
               "-I", os.path.join(ROOT, "include"), "-I", src_dir, "-c", os.path.join(src_dir, src),
               "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        subprocess.check_call(cmd)
        objs.append(obj)
    subprocess.check_call([hipbuild.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB, *objs])
    return LIB


def run(n_layers: int = 4, launches: int = 12) -> str:
    """Run the instrumented kernel over n_layers distinct stream layers cycled `launches` times
    (the first n_layers launches warm up) and return the Markdown summary."""
    import numpy as np
    import torch

    from bit_vector_lut_amd import synth, vqmlp

    if not os.path.exists(LIB):
        raise SystemExit("instrumented library missing: run the build step first")
    vqmlp.LIB_PATH = LIB
    vqmlp._lib = None
    vqmlp.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus > MAX_WG:
        raise SystemExit("%d compute units: the record area holds %d workgroups" % (cus, MAX_WG))
    mlps, xs = [], []
    for i in range(n_layers):
        L = synth.stream_layer(i)
        H, I, bh = L.H, L.I, L.had_block_h
        mlps.append(vqmlp.MLP.from_layer(L, t_max=8))
        xs.append(vqmlp.to_device(L.x))
        del L
        print("timeline: layer %d of %d uploaded" % (i + 1, n_layers), file=sys.stderr, flush=True)
    need = mlps[0].workspace_bytes(8)
    if need > REC_OFF:
        raise SystemExit("the forward's workspace (%d B) overlaps the records" % need)
    y = torch.empty_like(xs[0])
    ws = torch.zeros(REC_OFF + MAX_WG * REC_WORDS * 8, dtype=torch.uint8, device="cuda")
    recs = []
    for i in range(launches):
        ws[REC_OFF:].zero_()
        mlps[i % n_layers].forward(xs[i % n_layers], y, ws, path=1)
        torch.cuda.synchronize()
        if i >= n_layers:
            recs.append(ws[REC_OFF:].cpu().numpy().view(np.uint64)
                        .reshape(MAX_WG, REC_WORDS)[:cus].astype(np.int64))
    print("timeline: %d launches done" % launches, file=sys.stderr, flush=True)
    err = vqmlp.workspace_errors(ws)
    return summarize(recs, H // max(bh, 128 if H % 128 == 0 else 64), I // 32, err)


def summarize(recs, n_r, n_g, err) -> str:
    """Items are numbered as the kernel's queue numbers them: n_r input-rotation items (row
    chunks of the rotation block, at least 128 columns), then n_g gate/up items (one 32-row tile
    of both matrices each), then the down items."""
    import numpy as np

    lines = []
    spans, first_loop, ends = [], [], []
    per = {}
    nitems = []
    for d in recs:
        act = d[:, 0] > 0
        t0 = d[act, 0].min()
        spans.append((d[act, 1].max() - t0) / 100)
        ends += list((d[act, 1] - t0) / 100)
        for b in range(d.shape[0]):
            # an item counts once its products ran (the last barrier of the loop sees none)
            items = [int(d[b, 400 + j]) - 1 for j in range(8) if d[b, 400 + j] > 0 and d[b, 16 + 2 * j] > 0]
            nitems.append(len(items))
            for j, u in enumerate(items):
                st = np.array([d[b, 16 + 16 * w + 2 * j] for w in range(16)])
                en = np.array([d[b, 17 + 16 * w + 2 * j] for w in range(16)])
                if (st == 0).any() or (en == 0).any():
                    continue
                kind = "G" if u < n_r + n_g else "D"
                if j == 0:
                    first_loop.append((st.min() - t0) / 100)
                per.setdefault((kind, j), []).append(((st.min() - d[b, 2 + j]) / 100,
                                                      (st.max() - d[b, 2 + j]) / 100,
                                                      (en.max() - st.min()) / 100))
    lines.append("| launches | span median (us) | span min / max | first gate/up loop start, median (min / max) |")
    lines.append("|---|---|---|---|")
    lines.append("| %d | %.1f | %.1f / %.1f | %.1f (%.1f / %.1f) |" % (
        len(spans), np.median(spans), min(spans), max(spans), np.median(first_loop),
        min(first_loop), max(first_loop)))
    lines.append("")
    lines.append("Workgroup end times (us after the first workgroup's start), percentiles 10 / 50 / 90 / 100: "
                 "%.1f / %.1f / %.1f / %.1f.  Streaming items per workgroup: %s." % (
                     *np.percentile(ends, [10, 50, 90, 100]),
                     ", ".join("%d: %d" % (k, v) for k, v in sorted(
                         {k: nitems.count(k) // len(recs) for k in set(nitems)}.items()))))
    lines.append("")
    lines.append("| item (kind, position j) | count | barrier -> first wave's products (us) | "
                 "barrier -> last wave's products (us) | products, first wave start -> last wave end (us) |")
    lines.append("|---|---|---|---|---|")
    for key in sorted(per, key=lambda k: (k[1], k[0])):
        v = np.array(per[key])
        lines.append("| %s j=%d | %d | %.2f | %.2f | %.2f |" % (key[0], key[1], len(v), v[:, 0].mean(),
                                                               v[:, 1].mean(), v[:, 2].mean()))
    lines.append("")
    lines.append("Error word after the runs: %d (0 = every bounded wait ended normally)." % err)
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("step", choices=["build", "run"])
    ap.add_argument("--layers", type=int, default=4)
    args = ap.parse_args()
    if args.step == "build":
        print(build())
    else:
        sys.stdout.write(run(args.layers))


if __name__ == "__main__":
    main()
