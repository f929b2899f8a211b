// vqmlp_host.cpp -- host half of the VQ3 MLP library: argument checking, packing, plans,
// workspace carving and kernel dispatch.  Every public entry point is extern "C" and returns a
// vqmlp_status; failures set a per-thread message and launch nothing.
#include "internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "vqmlp.h"

using namespace vqmlp;

namespace {

thread_local std::string g_last_error;

vqmlp_status fail(vqmlp_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

}  // namespace

int vqmlp::set_last_error(int st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

namespace {

vqmlp_status ok() {
    g_last_error.clear();
    return VQMLP_OK;
}

vqmlp_status hip_fail(hipError_t e, const char* what) {
    return fail(VQMLP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// VQMLP_TRACE set to anything but "0": one line per call on stderr naming the kernels that the
// dispatch chose.  Read on every call (one getenv), so a process can switch it on and off.
bool trace_on() {
    const char* v = getenv("VQMLP_TRACE");
    return v && *v && strcmp(v, "0") != 0;
}

void trace(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    fprintf(stderr, "vqmlp: %s\n", buf);
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int default_block(int n) {
    int b = 1;
    while (b * 2 <= 128 && n % (b * 2) == 0) b *= 2;
    return b;
}

// ---------------------------------------------------------------- VQ3 packed layout

struct Layout {
    size_t codes_off, codes_bytes, cb_off, cb_bytes, sc_off, sc_bytes, total;
};

vqmlp_status check_shape(int N, int K) {
    if (N <= 0 || K <= 0 || N > (1 << 20) || K > (1 << 20))
        return fail(VQMLP_ERR_INVALID_ARG, "matrix shape %dx%d out of range", N, K);
    if (N % kTileRows)
        return fail(VQMLP_ERR_INVALID_ARG, "N=%d must be a multiple of %d", N, kTileRows);
    if (K % kTileCols)
        return fail(VQMLP_ERR_INVALID_ARG, "K=%d must be a multiple of %d", K, kTileCols);
    return VQMLP_OK;
}

Layout layout_of(int N, int K) {
    Layout L;
    L.codes_off = kHeaderBytes;
    L.codes_bytes = size_t(N / kTileRows) * (K / kTileCols) * kTileBytes;
    L.cb_off = align256(L.codes_off + L.codes_bytes);
    L.cb_bytes = size_t(N / kGroupRows) * kCodebook * 4;
    L.sc_off = align256(L.cb_off + L.cb_bytes);
    L.sc_bytes = size_t(N) * 2;
    L.total = align256(L.sc_off + L.sc_bytes);
    return L;
}

PackedHeader header_of(int N, int K, uint32_t kind, uint32_t entries, const Layout& L) {
    PackedHeader h;
    memset(&h, 0, sizeof h);
    h.magic = kMagic;
    h.version = VQMLP_LAYOUT_VERSION;
    h.N = uint32_t(N);
    h.K = uint32_t(K);
    h.group_rows = kGroupRows;
    h.entries = entries;
    h.kind = kind;
    h.codes_off = L.codes_off;
    h.codes_bytes = L.codes_bytes;
    h.cb_off = L.cb_off;
    h.cb_bytes = L.cb_bytes;
    h.sc_off = L.sc_off;
    h.sc_bytes = L.sc_bytes;
    h.total = L.total;
    return h;
}

vqmlp_status check_header(const PackedHeader& h, int N, int K, uint32_t kind, uint32_t entries,
                          const Layout& L, const char* name) {
    if (h.magic != kMagic)
        return fail(VQMLP_ERR_INVALID_ARG, "%s: bad magic 0x%08x (not a packed buffer)", name,
                    h.magic);
    if (h.version != VQMLP_LAYOUT_VERSION)
        return fail(VQMLP_ERR_INVALID_ARG, "%s: layout version %u, library expects %d", name,
                    h.version, VQMLP_LAYOUT_VERSION);
    if (int(h.N) != N || int(h.K) != K)
        return fail(VQMLP_ERR_INVALID_ARG, "%s: packed shape %ux%u, expected %dx%d", name, h.N,
                    h.K, N, K);
    if (h.kind != kind || h.entries != entries || h.group_rows != uint32_t(kGroupRows))
        return fail(VQMLP_ERR_INVALID_ARG, "%s: packed kind %u/%u entries, expected %u/%u", name,
                    h.kind, h.entries, kind, entries);
    if (h.codes_off != L.codes_off || h.cb_off != L.cb_off || h.sc_off != L.sc_off ||
        h.total != L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "%s: section offsets do not match the layout", name);
    return VQMLP_OK;
}

// code q of tile lane l: pair 16m + l%16, column 64k + 16*(q/4) + 4*(l/16) + q%4
inline unsigned get6(const uint8_t* lane12, int q) {
    const int bit = 6 * q;
    uint32_t w[3];
    memcpy(w, lane12, 12);
    const uint64_t lo = (uint64_t(w[1]) << 32) | w[0];
    const uint64_t hi = w[2];
    uint64_t v;
    if (bit + 6 <= 64)
        v = lo >> bit;
    else if (bit >= 64)
        v = hi >> (bit - 64);
    else
        v = (lo >> bit) | (hi << (64 - bit));
    return unsigned(v & 63);
}

VQ3View view_of(const void* packed, int N, int K) {
    const Layout L = layout_of(N, K);
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    VQ3View v;
    v.codes = base + L.codes_off;
    v.cb = reinterpret_cast<const uint32_t*>(base + L.cb_off);
    v.sc = reinterpret_cast<const uint16_t*>(base + L.sc_off);
    v.N = N;
    v.K = K;
    return v;
}

vqmlp_status read_device_header(const void* dev, PackedHeader* h, const char* name) {
    if (!dev) return fail(VQMLP_ERR_INVALID_ARG, "%s: null packed buffer", name);
    if (!aligned(dev, 256))
        return fail(VQMLP_ERR_INVALID_ARG, "%s: packed buffer must be 256-byte aligned", name);
    hipError_t e = hipMemcpy(h, dev, sizeof *h, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "reading a packed header");
    return VQMLP_OK;
}

vqmlp_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
        return fail(VQMLP_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950",
                    dev, p.gcnArchName);
    return VQMLP_OK;
}

}  // namespace

// ==================================================================== plan

struct FusedGeom {
    int tpw;                              // 0: the fused kernel does not take this shape
    int rc, fu, n_r, n_g, nsl, nqd, n_fu, total;
    size_t ctl_words;
};

struct vqmlp_plan {
    vqmlp_desc d;
    int bh, bi;
    VQ3View gate, up, down;
    FusedGeom fz;
    int cus;                              // compute units: workgroups of the fused kernel
    bool tiled_ok;
    bool vq2;                             // 2x16 matrices (vqmlp_create_vq2)
    int v2_ng, v2_nd;                     // 2x16 at T <= 8: K slices of gate/up and of down
                                          // (0: that path does not take the shape)
};

namespace {

// The gate/up product of the tiled path in 128-row by 128- (or 64-) token tiles: the first
// rows_main rows take whole rounds of workgroups on the CUs; the last rows_split rows, which
// would leave a partial round, are split along K into `splits` parts over the CUs.  With fewer
// tiles than CUs every row is split (rows_main = 0).  The rows left over after whole rounds run in
// 64-token tiles where the whole-K product's tiles hold 128 tokens (bm64): twice the workgroups,
// each with half the products, so that more CUs share the split rows and fewer planes are needed.
struct GateUpSplit {
    int rows_main, rows_split, splits, bm64;
};
GateUpSplit gateup_split(int I, int H, int T, int cus) {
    GateUpSplit g{I, 0, 1, 0};
    if (I % 128 || T <= kSkinnyT || cus <= 0) return g;
    const Vq3Tile t = T >= kVq3mmMinT ? vq3mm_tile(kGemmVQ3GateUpSplit, T) : Vq3Tile{64, 128};
    if (I % t.bn) return g;
    const int rt = I / t.bn, tt = (T + t.bm - 1) / t.bm, total = rt * tt;
    const int kt = H / 64;
    if (total < cus && T >= kVq3mmMinT) {
        // fewer tiles than CUs (the 64-row prefill chunk: 136 tiles): split every row's K so
        // that whole rounds of workgroups cover the CUs, each extra plane priced at 5%
        int best = 1;
        double best_cost = 1.0;
        for (int s = 2; s <= 8 && s <= kt / 8; ++s) {
            const double cost = double((total * s + cus - 1) / cus) / s + 0.05 * s;
            if (cost < best_cost - 1e-9) {
                best = s;
                best_cost = cost;
            }
        }
        if (best > 1) {
            g.rows_main = 0;
            g.rows_split = I;
            g.splits = best;
        }
        return g;
    }
    if (total <= cus || total % cus == 0) return g;
    const int main_rt = (total / cus) * cus / tt;
    const int bms = t.bm > 64 ? 64 : t.bm;  // tokens per tile of the split rows
    const int left = (rt - main_rt) * ((T + bms - 1) / bms);  // their tiles
    const int s = std::min(kt / 8, std::max(1, cus / left));
    if (main_rt <= 0 || s < 2) return g;
    g.rows_main = main_rt * t.bn;
    g.rows_split = I - g.rows_main;
    g.splits = s;
    g.bm64 = bms < t.bm && T >= kVq3mmMinT ? 1 : 0;
    return g;
}

struct Workspace {
    uint32_t* ctl;    // fused control block (zero before the first call, left zero by each)
    // fused region
    uint64_t* fxb;    // [2][8][H/2] tagged binary16 pairs
    uint64_t* fact;   // [8][I] tagged
    uint64_t* fab;    // [2][8][I/2] tagged binary16 pairs
    uint64_t* fpart;  // [nsl][8][H] tagged
    // tiled region
    uint16_t* xt;     // [T][H]
    float* a_t;       // [T][I]
    uint16_t* at;     // [T][I]
    float* dpart;     // [dsplit][T][H] partial sums of a K-split down projection
    int dsplit;
    float* gpart;     // [splits][T][2][rows] g, u partial sums of the K-split gate/up rows
    GateUpSplit gs;
    size_t bytes;
};

// The regions are disjoint: the fused kernel's tagged words must never see another path's
// data where it expects a tag.
Workspace carve(const vqmlp_plan* p, int T, void* base) {
    Workspace w;
    memset(&w, 0, sizeof w);
    const int H = p->d.H, I = p->d.I;
    size_t off = 0;
    auto take = [&](size_t n) {
        size_t o = off;
        off = align256(off + n);
        return o;
    };
    uint8_t* b = static_cast<uint8_t*>(base);
    const size_t o_ctl = take(std::max<size_t>(p->fz.ctl_words, kCtlHdr) * 4);
    const size_t o_fxb = take(2 * size_t(kSkinnyT) * H * 4);
    const size_t o_fact = take(size_t(kSkinnyT) * I * 8);
    const size_t o_fab = take(2 * size_t(kSkinnyT) * I * 4);
    const size_t o_fpart = take(size_t(std::max(p->fz.nsl, 1)) * kSkinnyT * H * 8);
    const int Tt = T > 0 ? T : 1;
    const size_t o_xt = take(size_t(Tt) * H * 2);
    const size_t o_at32 = take(size_t(Tt) * I * 4);
    const size_t o_at = take(size_t(Tt) * I * 2);
    int dsplit = T > kSkinnyT ? gemm_split(kGemmVQ3DownSplit, H, I, T, p->cus) : 1;
    GateUpSplit gs = T > kSkinnyT ? gateup_split(I, H, T, p->cus) : GateUpSplit{I, 0, 1};
    size_t gpart_bytes = gs.rows_split ? size_t(gs.splits) * Tt * 2 * gs.rows_split * 4 : 0;
    if (p->vq2 && T < kVq3mmMinT) {
        // 2x16 below the register-decode kernels: the tiled kernels (no leftover split of
        // gate/up) or, at T <= 8, the projection kernel's K slices: gate/up planes
        // [ng][T][2][I], down planes [nd][T][H].  From T = 33 a 2x16 plan takes the VQ3 rules.
        gs = GateUpSplit{I, 0, 1};
        gpart_bytes = 0;
        dsplit = gemm_split(kGemmVQ3DownSplit, H, I, T, p->cus);
        if (T <= kSkinnyT && p->v2_ng) {
            dsplit = p->v2_nd;
            gpart_bytes = size_t(p->v2_ng) * Tt * 2 * I * 4;
        }
    }
    const size_t o_dpart = take(dsplit > 1 ? size_t(dsplit) * Tt * H * 4 : 0);
    const size_t o_gpart = take(gpart_bytes);
    w.bytes = off;
    w.dsplit = dsplit;
    w.gs = gs;
    if (b) {
        w.dpart = reinterpret_cast<float*>(b + o_dpart);
        w.gpart = reinterpret_cast<float*>(b + o_gpart);
        w.ctl = reinterpret_cast<uint32_t*>(b + o_ctl);
        w.fxb = reinterpret_cast<uint64_t*>(b + o_fxb);
        w.fact = reinterpret_cast<uint64_t*>(b + o_fact);
        w.fab = reinterpret_cast<uint64_t*>(b + o_fab);
        w.fpart = reinterpret_cast<uint64_t*>(b + o_fpart);
        w.xt = reinterpret_cast<uint16_t*>(b + o_xt);
        w.a_t = reinterpret_cast<float*>(b + o_at32);
        w.at = reinterpret_cast<uint16_t*>(b + o_at);
    }
    return w;
}

// Item counts of the fused kernel for this shape (tpw = 0 when it does not apply).
FusedGeom fused_geom(int H, int I, int bh, int bi) {
    FusedGeom g;
    memset(&g, 0, sizeof g);
    g.tpw = fused_tpw(H);
    if (!g.tpw) return g;
    const int swt = kSkinnyWaves * g.tpw;  // K tiles per slice
    g.rc = std::max(bh, H % 128 == 0 ? 128 : 64);
    g.fu = std::max(bi, kTileRows);
    g.n_r = H / g.rc;
    g.n_g = I / kTileRows;
    g.nsl = (I / kTileCols + swt - 1) / swt;
    g.nqd = (H / kTileRows + 1) / 2;
    g.n_fu = I / g.fu;
    g.total = g.n_r + g.n_g + g.nsl * g.nqd;
    g.ctl_words = fused_ctl_words();
    // the kernel rotates rows of up to 256 columns in registers
    if (g.n_r > 1024 || g.rc > 256 || g.fu > 256) g.tpw = 0;
    return g;
}

vqmlp_status run_fused(const vqmlp_plan* p, int T, const void* x, void* y, const Workspace& w,
                       hipStream_t st) {
    const FusedGeom& g = p->fz;
    FusedArgs a;
    memset(&a, 0, sizeof a);
    a.gate = p->gate;
    a.up = p->up;
    a.down = p->down;
    a.H = p->d.H;
    a.I = p->d.I;
    a.T = T;
    a.bh = p->bh;
    a.bi = p->bi;
    a.rc = g.rc;
    a.fu = g.fu;
    a.n_r = g.n_r;
    a.n_g = g.n_g;
    a.nsl = g.nsl;
    a.nqd = g.nqd;
    a.n_fu = g.n_fu;
    a.total = g.total;
    a.norm_h = float(1.0 / std::sqrt(double(p->bh)));
    a.norm_i = float(1.0 / std::sqrt(double(p->bi)));
    a.x = static_cast<const uint16_t*>(x);
    a.s = p->d.s_in;
    a.sign_h = p->d.sign_h;
    a.sign_i = p->d.sign_i;
    a.y = static_cast<uint16_t*>(y);
    a.ctl = w.ctl;
    a.xb = w.fxb;
    a.act = w.fact;
    a.ab = w.fab;
    a.part = w.fpart;
    a.spin_limit = 1u << 18;
    a.dyn = 1;
    // one workgroup per CU, or one per streaming item when there are fewer (a small layer): the
    // others would only start and leave
    const int grid = std::max(1, std::min(p->cus, g.total - g.n_r));
    const hipError_t e = launch_fused(a, g.tpw, grid, st);
    if (e != hipSuccess) return hip_fail(e, "fused forward");
    return ok();
}

vqmlp_status run_tiled(const vqmlp_plan* p, int T, const void* x, void* y, const Workspace& w,
                       hipStream_t st) {
    const int H = p->d.H, I = p->d.I;
    hipError_t e = launch_rotate(T, H, p->bh, x, 0, p->d.s_in, p->d.sign_h, w.xt, 1, st);
    if (e != hipSuccess) return hip_fail(e, "rotate (input)");
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.vq2 = p->vq2 ? 1 : 0;
    g.N = I;
    g.K = H;
    g.T = T;
    g.x = w.xt;
    g.codes[0] = p->gate.codes;
    g.codes[1] = p->up.codes;
    g.cb[0] = p->gate.cb;
    g.cb[1] = p->up.cb;
    g.sc[0] = p->gate.sc;
    g.sc[1] = p->up.sc;
    g.sign = p->d.sign_i;
    // the gate/up epilogue rotates a itself when a rotation block is one 128-row tile
    const bool fused_rot = p->bi == 128 && I % 128 == 0;
    const GateUpSplit& gs = w.gs;
    g.N = gs.rows_main;
    g.ldo = I;
    g.norm = float(1.0 / 11.313708498984761);  // 1/sqrt(128)
    g.kind = fused_rot ? kGemmVQ3GateUpRot : kGemmVQ3GateUp;
    g.out16 = w.at;
    g.out32 = w.a_t;
    if (gs.rows_main > 0) {
        e = launch_gemm(g, st);
        if (e != hipSuccess) return hip_fail(e, "tiled gate/up");
    }
    if (gs.rows_split) {
        // the rows that would leave a partial round of workgroups: K split over the CUs, then
        // one pass that sums the parts and applies the same epilogue
        const int r0 = gs.rows_main;
        GemmArgs q = g;
        q.kind = kGemmVQ3GateUpSplit;
        q.N = gs.rows_split;
        q.ldo = 0;
        q.ksplit = gs.splits;
        q.bm64 = gs.bm64;
        for (int m = 0; m < 2; ++m) {
            // row r0 of the packed codes and codebooks (VQ3 tiles, or 2x16 pair rows of H / 8
            // words and 16 centroids per 8 rows)
            q.codes[m] = p->vq2 ? g.codes[m] + size_t(r0 / 2) * (H / 2)
                                : g.codes[m] + size_t(r0 / kTileRows) * (H / kTileCols) * kTileBytes;
            q.cb[m] = g.cb[m] + size_t(r0 / 8) * (p->vq2 ? 16 : 64);
            q.sc[m] = g.sc[m] + r0;
        }
        q.sign = nullptr;
        q.norm = 1.f;  // unscaled planes
        q.out32 = w.gpart;
        e = launch_gemm(q, st);
        if (e != hipSuccess) return hip_fail(e, "tiled gate/up (K split)");
        e = launch_gateup_combine(T, gs.rows_split, gs.splits, w.gpart, p->gate.sc + r0,
                                  p->up.sc + r0, p->d.sign_i ? p->d.sign_i + r0 : nullptr,
                                  fused_rot ? 1 : 0, g.norm, I, w.at + r0, w.a_t + r0, st);
        if (e != hipSuccess) return hip_fail(e, "gate/up split combine");
    }
    if (!fused_rot) {
        e = launch_rotate(T, I, p->bi, w.a_t, 1, nullptr, nullptr, w.at, 1, st);
        if (e != hipSuccess) return hip_fail(e, "rotate (intermediate)");
    }
    GemmArgs d;
    memset(&d, 0, sizeof d);
    d.vq2 = p->vq2 ? 1 : 0;
    d.kind = kGemmVQ3Down;
    d.N = H;
    d.K = I;
    d.T = T;
    d.x = w.at;
    d.codes[0] = p->down.codes;
    d.cb[0] = p->down.cb;
    d.sc[0] = p->down.sc;
    d.out16 = static_cast<uint16_t*>(y);
    if (w.dsplit > 1) {
        // too few row tiles to fill the CUs: split K, then sum the planes and scale
        d.kind = kGemmVQ3DownSplit;
        d.ksplit = w.dsplit;
        d.norm = 1.f;  // unscaled planes
        d.out32 = w.dpart;
        e = launch_gemm(d, st);
        if (e != hipSuccess) return hip_fail(e, "tiled down (K split)");
        e = launch_split_reduce(T, H, w.dsplit, w.dpart, p->down.sc, static_cast<uint16_t*>(y), st);
        if (e != hipSuccess) return hip_fail(e, "down split reduction");
        return ok();
    }
    e = launch_gemm(d, st);
    if (e != hipSuccess) return hip_fail(e, "tiled down");
    return ok();
}

// The trace line of a forward on the tiled / register-decode kernels.
void trace_tiled(const vqmlp_plan* p, int T, const Workspace& w) {
    const char* fam = T >= kVq3mmMinT ? "register-decode" : "tiled";
    char split[96] = "";
    if (w.gs.rows_split)
        snprintf(split, sizeof split, ", rows %d.. K-split %d ways%s + combine", w.gs.rows_main,
                 w.gs.splits, w.gs.bm64 ? " in 64-token tiles" : "");
    char dsplit[64] = "";
    if (w.dsplit > 1) snprintf(dsplit, sizeof dsplit, " K-split %d ways + reduction", w.dsplit);
    trace("forward%s H=%d I=%d T=%d: input rotation; %s gate/up on rows 0..%d%s; %s; %s down%s",
          p->vq2 ? " 2x16" : "", p->d.H, p->d.I, T, fam, w.gs.rows_main, split,
          p->bi == 128 && p->d.I % 128 == 0 ? "intermediate rotation in the gate/up epilogue"
                                           : "intermediate rotation kernel",
          fam, dsplit);
}

// 2x16 matrices at T <= 8: rotate x, the gate and up products as unscaled FP32 planes (K
// slices of at most kVq2MaxK columns), a = silu(g) u sign with its rotation, the down product
// (K slices), the slice sum scaled into y.
vqmlp_status run_vq2_skinny(const vqmlp_plan* p, int T, const void* x, void* y,
                            const Workspace& w, hipStream_t st) {
    const int H = p->d.H, I = p->d.I, ng = p->v2_ng, nd = p->v2_nd;
    hipError_t e = launch_rotate(T, H, p->bh, x, 0, p->d.s_in, p->d.sign_h, w.xt, 1, st);
    if (e != hipSuccess) return hip_fail(e, "rotate (input)");
    Vq2Args a;
    memset(&a, 0, sizeof a);
    a.x = w.xt;
    a.N = I;
    a.K = H / ng;
    a.T = T;
    a.ldk = H;
    a.nsplit = ng;
    a.o32_t = 2 * I;
    a.o32_s = T * 2 * I;
    // gate and up in one launch: planes [slice][t][g | u]
    a.codes = reinterpret_cast<const uint32_t*>(p->gate.codes);
    a.cb = p->gate.cb;
    a.sc = p->gate.sc;
    a.codes2 = reinterpret_cast<const uint32_t*>(p->up.codes);
    a.cb2 = p->up.cb;
    a.sc2 = p->up.sc;
    a.o32_m = I;
    a.out32 = w.gpart;
    e = launch_vq2_8(a, st);
    if (e != hipSuccess) return hip_fail(e, "2x16 gate/up");
    const bool rot128 = p->bi == 128;
    e = launch_gateup_combine(T, I, ng, w.gpart, p->gate.sc, p->up.sc, p->d.sign_i,
                              rot128 ? 1 : 0, float(1.0 / std::sqrt(128.0)), I, w.at, w.a_t, st);
    if (e != hipSuccess) return hip_fail(e, "2x16 gate/up combine");
    if (!rot128) {
        e = launch_rotate(T, I, p->bi, w.a_t, 1, nullptr, nullptr, w.at, 1, st);
        if (e != hipSuccess) return hip_fail(e, "rotate (intermediate)");
    }
    Vq2Args d;
    memset(&d, 0, sizeof d);
    d.codes = reinterpret_cast<const uint32_t*>(p->down.codes);
    d.cb = p->down.cb;
    d.sc = p->down.sc;
    d.x = w.at;
    d.N = H;
    d.K = I / nd;
    d.T = T;
    d.ldk = I;
    d.nsplit = nd;
    if (nd > 1) {
        d.out32 = w.dpart;
        d.o32_t = H;
        d.o32_s = T * H;
    } else {
        d.y = static_cast<uint16_t*>(y);
    }
    e = launch_vq2_8(d, st);
    if (e != hipSuccess) return hip_fail(e, "2x16 down");
    if (nd > 1) {
        e = launch_split_reduce(T, H, nd, w.dpart, p->down.sc, static_cast<uint16_t*>(y), st);
        if (e != hipSuccess) return hip_fail(e, "2x16 down slice sum");
    }
    return ok();
}

// Validate one packed VQ3 matrix (header read through a synchronous copy) and view it.
vqmlp_status vq3_view_checked(const void* dev, int N, int K, const char* name, VQ3View* v) {
    PackedHeader h;
    vqmlp_status st;
    if ((st = read_device_header(dev, &h, name))) return st;
    if ((st = check_header(h, N, K, 0, kCodebook, layout_of(N, K), name))) return st;
    *v = view_of(dev, N, K);
    return VQMLP_OK;
}

using ViewChecked = vqmlp_status (*)(const void*, int, int, const char*, VQ3View*);
int vq2_slices(int K);

// The plan of either format: shapes, blocks, pointers, device, headers (view_checked).
vqmlp_status create_plan(const vqmlp_desc* desc, vqmlp_plan** out, bool vq2,
                         ViewChecked view_checked) {
    if (!desc || !out) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_create: null pointer");
    *out = nullptr;
    const vqmlp_desc& d = *desc;
    vqmlp_status st;
    if ((st = check_shape(d.I, d.H))) return st;  // gate/up: N = I, K = H
    if ((st = check_shape(d.H, d.I))) return st;  // down:    N = H, K = I
    if (d.t_max < 0 || d.t_max > (1 << 20))
        return fail(VQMLP_ERR_INVALID_ARG, "t_max=%d out of range", d.t_max);
    const int bh = d.had_block_h ? d.had_block_h : default_block(d.H);
    const int bi = d.had_block_i ? d.had_block_i : default_block(d.I);
    if (!is_pow2(bh) || bh < 2 || bh > 1024 || d.H % bh)
        return fail(VQMLP_ERR_INVALID_ARG, "Hadamard block %d does not divide H=%d", bh, d.H);
    if (!is_pow2(bi) || bi < 2 || bi > 1024 || d.I % bi)
        return fail(VQMLP_ERR_INVALID_ARG, "Hadamard block %d does not divide I=%d", bi, d.I);
    if (!d.s_in) return fail(VQMLP_ERR_INVALID_ARG, "s_in is NULL");
    if (!aligned(d.s_in, 16) || (d.sign_h && !aligned(d.sign_h, 16)) ||
        (d.sign_i && !aligned(d.sign_i, 16)))
        return fail(VQMLP_ERR_INVALID_ARG, "s_in / sign pointers must be 16-byte aligned");
    if ((st = check_device())) return st;
    noalloc_setup();  // the allocation-free forward's scratch array on this device (once)
    VQ3View vg, vu, vd;
    if ((st = view_checked(d.gate, d.I, d.H, "gate", &vg))) return st;
    if ((st = view_checked(d.up, d.I, d.H, "up", &vu))) return st;
    if ((st = view_checked(d.down, d.H, d.I, "down", &vd))) return st;
    vqmlp_plan* p = new (std::nothrow) vqmlp_plan;
    if (!p) return fail(VQMLP_ERR_INVALID_ARG, "out of host memory");
    p->d = d;
    p->bh = bh;
    p->bi = bi;
    p->gate = vg;
    p->up = vu;
    p->down = vd;
    p->vq2 = vq2;
    if (vq2) {
        memset(&p->fz, 0, sizeof p->fz);  // the fused kernel reads the three-bit tiles only
        const bool ok_i = d.I % 128 == 0;  // the gate/up combine pass rotates 128-row blocks
        p->v2_ng = ok_i ? vq2_slices(d.H) : 0;
        p->v2_nd = ok_i ? vq2_slices(d.I) : 0;
    } else {
        p->fz = fused_geom(d.H, d.I, bh, bi);
        p->v2_ng = p->v2_nd = 0;
    }
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        p->cus = cus;
    }
    p->tiled_ok = d.H % 64 == 0 && d.I % 64 == 0;
    *out = p;
    return ok();
}

// K slices of at most kVq2MaxK columns, each a multiple of 32 (0: none fits)
int vq2_slices(int K) {
    for (int s = 1; s <= 64; ++s)
        if (K % s == 0 && (K / s) % 32 == 0 && K / s <= kVq2MaxK) return s;
    return 0;
}

}  // namespace

// ==================================================================== extern "C"

extern "C" {

int vqmlp_abi_version(void) { return VQMLP_ABI_VERSION; }

const char* vqmlp_last_error(void) { return g_last_error.c_str(); }

vqmlp_status vqmlp_packed_bytes(int N, int K, size_t* bytes) {
    if (!bytes) return fail(VQMLP_ERR_INVALID_ARG, "bytes is NULL");
    vqmlp_status st = check_shape(N, K);
    if (st) return st;
    *bytes = layout_of(N, K).total;
    return ok();
}

vqmlp_status vqmlp_pack(int N, int K, const uint8_t* codes, const uint16_t* codebook,
                        const uint16_t* row_scale, void* packed, size_t packed_bytes) {
    vqmlp_status st = check_shape(N, K);
    if (st) return st;
    if (!codes || !codebook || !row_scale || !packed)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_pack: null pointer");
    const Layout L = layout_of(N, K);
    if (packed_bytes < L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_pack: buffer holds %zu bytes, needs %zu",
                    packed_bytes, L.total);
    const size_t ncodes = size_t(N / 2) * K;
    for (size_t i = 0; i < ncodes; ++i)
        if (codes[i] > 63)
            return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_pack: code %u at pair %zu column %zu > 63",
                        codes[i], i / K, i % K);
    uint8_t* out = static_cast<uint8_t*>(packed);
    memset(out, 0, L.total);
    PackedHeader h = header_of(N, K, 0, kCodebook, L);
    memcpy(out, &h, sizeof h);
    const int MT = N / kTileRows, KT = K / kTileCols;
    uint8_t* tiles = out + L.codes_off;
    for (int m = 0; m < MT; ++m)
        for (int k = 0; k < KT; ++k) {
            uint8_t* tile = tiles + (size_t(m) * KT + k) * kTileBytes;
            for (int l = 0; l < 64; ++l) {
                const int pair = m * kTilePairs + (l % 16);
                const uint8_t* c = codes + size_t(pair) * K + size_t(k) * kTileCols + 4 * (l / 16);
                // 16 codes: q = 4s + i at bits 6q..6q+5 of a 96-bit little-endian word
                uint64_t lo = 0, hi = 0;
                for (int q = 0; q < 16; ++q) {
                    const uint64_t v = c[16 * (q / 4) + (q % 4)];
                    const int bit = 6 * q;
                    if (bit + 6 <= 64) {
                        lo |= v << bit;
                    } else if (bit >= 64) {
                        hi |= v << (bit - 64);
                    } else {
                        lo |= v << bit;
                        hi |= v >> (64 - bit);
                    }
                }
                const uint32_t w[3] = {uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi)};
                memcpy(tile + 12 * l, w, 12);
            }
        }
    memcpy(out + L.cb_off, codebook, L.cb_bytes);
    memcpy(out + L.sc_off, row_scale, L.sc_bytes);
    return ok();
}

vqmlp_status vqmlp_unpack(int N, int K, const void* packed, size_t packed_bytes, uint8_t* codes,
                          uint16_t* codebook, uint16_t* row_scale) {
    vqmlp_status st = check_shape(N, K);
    if (st) return st;
    if (!packed || !codes || !codebook || !row_scale)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_unpack: null pointer");
    const Layout L = layout_of(N, K);
    if (packed_bytes < L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_unpack: buffer holds %zu bytes, needs %zu",
                    packed_bytes, L.total);
    const uint8_t* in = static_cast<const uint8_t*>(packed);
    PackedHeader h;
    memcpy(&h, in, sizeof h);
    st = check_header(h, N, K, 0, kCodebook, L, "vqmlp_unpack");
    if (st) return st;
    const int MT = N / kTileRows, KT = K / kTileCols;
    const uint8_t* tiles = in + L.codes_off;
    for (int m = 0; m < MT; ++m)
        for (int k = 0; k < KT; ++k) {
            const uint8_t* tile = tiles + (size_t(m) * KT + k) * kTileBytes;
            for (int l = 0; l < 64; ++l) {
                const int pair = m * kTilePairs + (l % 16);
                for (int q = 0; q < 16; ++q) {
                    const int col = k * kTileCols + 16 * (q / 4) + 4 * (l / 16) + (q % 4);
                    codes[size_t(pair) * K + col] = uint8_t(get6(tile + 12 * l, q));
                }
            }
        }
    memcpy(codebook, in + L.cb_off, L.cb_bytes);
    memcpy(row_scale, in + L.sc_off, L.sc_bytes);
    return ok();
}

vqmlp_status vqmlp_dequant(int N, int K, const void* packed, float* w, void* stream) {
    vqmlp_status st = check_shape(N, K);
    if (st) return st;
    if (!w) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_dequant: null output");
    st = check_device();
    if (st) return st;
    PackedHeader h;
    st = read_device_header(packed, &h, "vqmlp_dequant");
    if (st) return st;
    st = check_header(h, N, K, 0, kCodebook, layout_of(N, K), "vqmlp_dequant");
    if (st) return st;
    hipError_t e = launch_dequant(view_of(packed, N, K), w, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    return ok();
}

vqmlp_status vqmlp_rotate(int T, int n, int b, const uint16_t* x, const uint16_t* s,
                          const int8_t* sign, float* out, void* stream) {
    if (T < 0 || n <= 0 || !is_pow2(b) || b < 2 || b > 1024 || n % b)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_rotate: bad shape T=%d n=%d b=%d", T, n, b);
    if (T == 0) return ok();
    if (!x || !out) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_rotate: null pointer");
    vqmlp_status st = check_device();
    if (st) return st;
    hipError_t e = launch_rotate(T, n, b, x, 0, s, sign, out, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "rotate launch");
    return ok();
}

vqmlp_status vqmlp_create(const vqmlp_desc* desc, vqmlp_plan** out) {
    return create_plan(desc, out, false, vq3_view_checked);
}

vqmlp_status vqmlp_destroy(vqmlp_plan* plan) {
    delete plan;
    return ok();
}

vqmlp_status vqmlp_workspace_bytes(const vqmlp_plan* p, int T, size_t* bytes) {
    if (!p || !bytes) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_workspace_bytes: null pointer");
    if (T < 0 || T > p->d.t_max)
        return fail(VQMLP_ERR_INVALID_ARG, "T=%d outside [0, t_max=%d]", T, p->d.t_max);
    *bytes = carve(p, T, nullptr).bytes;
    return ok();
}

vqmlp_status vqmlp_forward_path(const vqmlp_plan* p, int T, const void* x, void* y,
                                void* workspace, size_t workspace_bytes, int path,
                                void* stream) {
    if (!p) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_forward: null plan");
    if (T < 0 || T > p->d.t_max)
        return fail(VQMLP_ERR_INVALID_ARG, "T=%d outside [0, t_max=%d]", T, p->d.t_max);
    if (path < 0 || path > 2) return fail(VQMLP_ERR_INVALID_ARG, "unknown path %d", path);
    if (T == 0) return ok();
    if (!x || !y || !workspace) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_forward: null pointer");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256))
        return fail(VQMLP_ERR_INVALID_ARG,
                    "x and y must be 16-byte aligned, the workspace 256-byte aligned");
    const Workspace w = carve(p, T, workspace);
    if (workspace_bytes < w.bytes)
        return fail(VQMLP_ERR_WORKSPACE, "workspace holds %zu bytes, this forward needs %zu",
                    workspace_bytes, w.bytes);
    const uint8_t* wb = static_cast<const uint8_t*>(workspace);
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    const uint8_t* yb = static_cast<const uint8_t*>(y);
    const size_t xy = size_t(T) * p->d.H * 2;
    if ((xb < wb + w.bytes && wb < xb + xy) || (yb < wb + w.bytes && wb < yb + xy))
        return fail(VQMLP_ERR_INVALID_ARG, "x or y overlaps the workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p->vq2) {
        // 1: the 2x16 projection kernels (T <= 8), 2: the tiled kernels; 0 picks the first for
        // T <= 8 where they apply
        const bool skinny = p->v2_ng > 0 && p->v2_nd > 0;
        if (path == 1 && (T > kSkinnyT || !skinny))
            return fail(VQMLP_ERR_UNSUPPORTED,
                        "the 2x16 T <= 8 path takes T <= %d and I a multiple of 128 (T=%d)",
                        kSkinnyT, T);
        const int use = path == 0 ? (T <= kSkinnyT && skinny ? 1 : 2) : path;
        if (use == 1) {
            if (trace_on())
                trace("forward 2x16 H=%d I=%d T=%d: input rotation; 2x16 projection kernel, gate "
                      "and up in one launch (%d K slices); gate/up combine; down (%d K slices)%s",
                      p->d.H, p->d.I, T, p->v2_ng, p->v2_nd, p->v2_nd > 1 ? " + slice sum" : "");
            return run_vq2_skinny(p, T, x, y, w, st);
        }
        if (!p->tiled_ok)
            return fail(VQMLP_ERR_UNSUPPORTED, "the tiled path takes H and I multiples of 64");
        if (trace_on()) trace_tiled(p, T, w);
        return run_tiled(p, T, x, y, w, st);
    }
    // 1: the fused single-launch kernel (T <= 8), 2: the tiled kernels; 0 picks the fused
    // kernel for T <= 8 where it applies, else the tiled kernels
    const bool fused_ok = p->fz.tpw > 0;
    if (path == 1) {
        if (T > kSkinnyT)
            return fail(VQMLP_ERR_UNSUPPORTED, "the fused kernel takes T <= %d (T=%d)", kSkinnyT, T);
        if (!fused_ok)
            return fail(VQMLP_ERR_UNSUPPORTED, "the fused kernel takes H <= %d (H=%d)",
                        kSkinnyWaves * kSkinnyMaxTPW * kTileCols, p->d.H);
    }
    const int use = path == 0 ? (T <= kSkinnyT && fused_ok ? 1 : 2) : path;
    if (use == 2 && !p->tiled_ok)
        return fail(VQMLP_ERR_UNSUPPORTED, "the tiled path takes H and I multiples of 64");
    if (use == 1) {
        if (trace_on())
            trace("forward H=%d I=%d T=%d: fused kernel (%d tiles per wave, %d workgroups; items: "
                  "%d input rotation, %d gate/up, %d down in %d K slices)",
                  p->d.H, p->d.I, T, p->fz.tpw, std::max(1, std::min(p->cus, p->fz.total - p->fz.n_r)),
                  p->fz.n_r, p->fz.n_g,
                  p->fz.nsl * p->fz.nqd, p->fz.nsl);
        return run_fused(p, T, x, y, w, st);
    }
    if (trace_on()) trace_tiled(p, T, w);
    return run_tiled(p, T, x, y, w, st);
}

vqmlp_status vqmlp_forward(const vqmlp_plan* p, int T, const void* x, void* y, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return vqmlp_forward_path(p, T, x, y, workspace, workspace_bytes, 0, stream);
}

vqmlp_status vqmlp_workspace_errors(void* workspace, size_t workspace_bytes, int clear,
                                    uint32_t* bits, void* stream) {
    if (!workspace || !bits) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_workspace_errors: null pointer");
    if (!aligned(workspace, 256) || workspace_bytes < kCtlHdr * 4)
        return fail(VQMLP_ERR_INVALID_ARG,
                    "vqmlp_workspace_errors: the workspace must be 256-byte aligned and hold "
                    "at least %d bytes", int(kCtlHdr * 4));
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t* err = static_cast<uint32_t*>(workspace) + kCtlError;  // control block at offset 0
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "vqmlp_workspace_errors: stream synchronisation");
    uint32_t v = 0;
    e = hipMemcpy(&v, err, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "vqmlp_workspace_errors: reading the error word");
    if (clear && v) {
        e = hipMemsetAsync(err, 0, sizeof v, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "vqmlp_workspace_errors: clearing the error word");
    }
    *bits = v;
    return ok();
}

vqmlp_status vqmlp_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_stream_read: null pointer");
    if (!aligned(buf, 16) || bytes % 16)
        return fail(VQMLP_ERR_INVALID_ARG,
                    "vqmlp_stream_read: buf must be 16-byte aligned and bytes a multiple of 16");
    vqmlp_status st = check_device();
    if (st) return st;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    hipError_t e = launch_stream_read(buf, bytes, sink, cus, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stream read launch");
    return ok();
}

// ------------------------------------------------------------------ scalar-LUT projection

static vqmlp_status lut_shape(int bits, int N, int K) {
    if (bits != 2 && bits != 4) return fail(VQMLP_ERR_INVALID_ARG, "bits=%d (2 or 4)", bits);
    if (N <= 0 || K <= 0 || N > (1 << 20) || K > (1 << 20) || N % 64 || K % 64)
        return fail(VQMLP_ERR_INVALID_ARG, "LUT matrix %dx%d: both must be multiples of 64", N, K);
    return VQMLP_OK;
}

static Layout lut_layout(int bits, int N, int K) {
    Layout L;
    L.codes_off = kHeaderBytes;
    L.codes_bytes = size_t(N) * K * bits / 8;
    L.cb_off = align256(L.codes_off + L.codes_bytes);
    L.cb_bytes = size_t(N / 8) * (1u << bits) * 2;
    L.sc_off = align256(L.cb_off + L.cb_bytes);
    L.sc_bytes = size_t(N) * 2;
    L.total = align256(L.sc_off + L.sc_bytes);
    return L;
}

vqmlp_status vqmlp_lut_packed_bytes(int bits, int N, int K, size_t* bytes) {
    if (!bytes) return fail(VQMLP_ERR_INVALID_ARG, "bytes is NULL");
    vqmlp_status st = lut_shape(bits, N, K);
    if (st) return st;
    *bytes = lut_layout(bits, N, K).total;
    return ok();
}

vqmlp_status vqmlp_lut_pack(int bits, int N, int K, const uint8_t* codes, const uint16_t* lut,
                            const uint16_t* row_scale, void* packed, size_t bytes) {
    vqmlp_status st = lut_shape(bits, N, K);
    if (st) return st;
    if (!codes || !lut || !row_scale || !packed)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_pack: null pointer");
    const Layout L = lut_layout(bits, N, K);
    if (bytes < L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_pack: buffer holds %zu bytes, needs %zu",
                    bytes, L.total);
    const unsigned lim = 1u << bits;
    for (size_t i = 0; i < size_t(N) * K; ++i)
        if (codes[i] >= lim)
            return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_pack: code %u >= %u at %zu", codes[i],
                        lim, i);
    uint8_t* out = static_cast<uint8_t*>(packed);
    memset(out, 0, L.total);
    PackedHeader h = header_of(N, K, uint32_t(bits), lim, L);
    memcpy(out, &h, sizeof h);
    const int per = 32 / bits;
    uint32_t* words = reinterpret_cast<uint32_t*>(out + L.codes_off);
    for (int n = 0; n < N; ++n)
        for (int j = 0; j < K; ++j)
            words[(size_t(n) * K + j) / per] |= uint32_t(codes[size_t(n) * K + j])
                                                << (bits * (j % per));
    memcpy(out + L.cb_off, lut, L.cb_bytes);
    memcpy(out + L.sc_off, row_scale, L.sc_bytes);
    return ok();
}

vqmlp_status vqmlp_lut_unpack(int bits, int N, int K, const void* packed, size_t bytes,
                              uint8_t* codes, uint16_t* lut, uint16_t* row_scale) {
    vqmlp_status st = lut_shape(bits, N, K);
    if (st) return st;
    if (!packed || !codes || !lut || !row_scale)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_unpack: null pointer");
    const Layout L = lut_layout(bits, N, K);
    if (bytes < L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_unpack: buffer holds %zu bytes, needs %zu",
                    bytes, L.total);
    const uint8_t* in = static_cast<const uint8_t*>(packed);
    PackedHeader h;
    memcpy(&h, in, sizeof h);
    st = check_header(h, N, K, uint32_t(bits), 1u << bits, L, "vqmlp_lut_unpack");
    if (st) return st;
    const int per = 32 / bits;
    const uint32_t* words = reinterpret_cast<const uint32_t*>(in + L.codes_off);
    for (int n = 0; n < N; ++n)
        for (int j = 0; j < K; ++j)
            codes[size_t(n) * K + j] = uint8_t(
                (words[(size_t(n) * K + j) / per] >> (bits * (j % per))) & ((1u << bits) - 1));
    memcpy(lut, in + L.cb_off, L.cb_bytes);
    memcpy(row_scale, in + L.sc_off, L.sc_bytes);
    return ok();
}

// The scalar-LUT forward has no plan; its K splits assume this many CUs (MI355X), so that the
// workspace size does not depend on the device.
constexpr int kLutSplitCUs = 256;

vqmlp_status vqmlp_lut_workspace_bytes(int N, int K, int T, int r, size_t* bytes) {
    if (!bytes) return fail(VQMLP_ERR_INVALID_ARG, "bytes is NULL");
    if (N <= 0 || K <= 0 || T < 0 || r < 0 || r > 256)
        return fail(VQMLP_ERR_INVALID_ARG, "bad LUT workspace query");
    const size_t Tt = T ? T : 1;
    const int zs = gemm_split(kGemmDense32, r ? r : 1, K, T, kLutSplitCUs);
    const int ls = gemm_split(kGemmLUT2, N, K, T, kLutSplitCUs);  // same split for both widths
    *bytes = align256(Tt * K * 2) + align256(Tt * (r ? r : 1) * 4) +
             (zs > 1 ? align256(size_t(zs) * Tt * (r ? r : 1) * 4) : 0) +
             (ls > 1 ? align256(size_t(ls) * Tt * N * 4) : 0) + 256;
    // T <= 8: x~ and the per-chunk partial sums of z (at most K / 64 chunks of 8 rows), or the
    // argmax head's per-workgroup bests
    if (T <= kSkinnyT)
        *bytes = std::max(*bytes, align256(Tt * K * 2) +
                                      std::max(align256(size_t(K / 64 + 1) * kSkinnyT * (r ? r : 1) * 4),
                                               align256(size_t(kArgmaxMaxGroups) * kSkinnyT * 8)) +
                                      256);
    return ok();
}

}  // extern "C"

// A validated scalar-LUT projection: everything a forward needs but its rows.
struct vqmlp_lut_plan {
    int bits, N, K, r, had_block;
    int cus;  // compute units of the device at creation (workgroups of the argmax head)
    const uint8_t* base;
    Layout L;
    const uint16_t *U, *V, *s;
    const int8_t* sign;
};

namespace {

// shapes, rank and block: the checks that need no device
vqmlp_status lut_args(int bits, int N, int K, int r, int had_block) {
    vqmlp_status st = lut_shape(bits, N, K);
    if (st) return st;
    if (r < 0 || r > 256) return fail(VQMLP_ERR_INVALID_ARG, "scalar-LUT projection: r=%d", r);
    if (had_block && (!is_pow2(had_block) || had_block < 2 || had_block > 1024 || K % had_block))
        return fail(VQMLP_ERR_INVALID_ARG, "Hadamard block %d does not divide K=%d", had_block, K);
    return VQMLP_OK;
}

vqmlp_status lut_validate(int bits, int N, int K, const void* packed, const uint16_t* U,
                          const uint16_t* V, int r, const uint16_t* s, const int8_t* sign,
                          int had_block, vqmlp_lut_plan* p) {
    vqmlp_status st = lut_args(bits, N, K, r, had_block);
    if (st) return st;
    if (!packed) return fail(VQMLP_ERR_INVALID_ARG, "scalar-LUT projection: null packed buffer");
    if (r > 0 && (!U || !V))
        return fail(VQMLP_ERR_INVALID_ARG, "scalar-LUT projection: r=%d needs U and V", r);
    if ((U && !aligned(U, 16)) || (V && !aligned(V, 16)))
        return fail(VQMLP_ERR_INVALID_ARG, "U, V must be 16-byte aligned");
    if ((st = check_device())) return st;
    const Layout L = lut_layout(bits, N, K);
    PackedHeader h;
    if ((st = read_device_header(packed, &h, "lut"))) return st;
    if ((st = check_header(h, N, K, uint32_t(bits), 1u << bits, L, "lut"))) return st;
    p->bits = bits;
    p->N = N;
    p->K = K;
    p->r = r;
    p->had_block = had_block;
    p->base = static_cast<const uint8_t*>(packed);
    p->L = L;
    p->U = U;
    p->V = V;
    p->s = s;
    p->sign = sign;
    return VQMLP_OK;
}

vqmlp_status lut_run(const vqmlp_lut_plan& p, int T, const void* x, void* y, void* workspace,
                     size_t workspace_bytes, void* stream) {
    const int N = p.N, K = p.K, r = p.r;
    if (T < 0) return fail(VQMLP_ERR_INVALID_ARG, "scalar-LUT projection: T=%d", T);
    if (T == 0) return ok();
    if (!x || !y || !workspace)
        return fail(VQMLP_ERR_INVALID_ARG, "scalar-LUT projection: null pointer");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256))
        return fail(VQMLP_ERR_INVALID_ARG, "x, y must be 16-byte aligned, the workspace 256");
    size_t need = 0;
    vqmlp_lut_workspace_bytes(N, K, T, r, &need);
    if (workspace_bytes < need)
        return fail(VQMLP_ERR_WORKSPACE, "workspace holds %zu bytes, this forward needs %zu",
                    workspace_bytes, need);
    const Layout& L = p.L;
    uint8_t* wb = static_cast<uint8_t*>(workspace) + 256;
    uint16_t* xt = reinterpret_cast<uint16_t*>(wb);
    float* z = reinterpret_cast<float*>(wb + align256(size_t(T) * K * 2));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint8_t* base = p.base;
    const uint16_t *U = p.U, *V = p.V;
    const int bits = p.bits;
    const int hb = p.had_block ? p.had_block : 1;
    if (T <= kSkinnyT && K <= kLut8MaxK && r % 16 == 0 && lut8_chunk(K, hb) >= 64 &&
        aligned(p.s, 16) && aligned(p.sign, 8)) {  // (the pre-pass reads s and sign in vectors)
        // decode-size T: one pre-pass (rotation and per-chunk partial sums of z), then the
        // code-stream kernel (its epilogue adds U z in FP32)
        if (trace_on())
            trace("scalar-LUT %d-bit N=%d K=%d T=%d r=%d: pre-pass (rotation, %d planes of z), "
                  "code-stream kernel", bits, N, K, T, r, lut8_planes(K, hb));
        float* zp = reinterpret_cast<float*>(wb + align256(size_t(T) * K * 2));
        hipError_t e = launch_lut8_pre(T, K, hb, static_cast<const uint16_t*>(x), p.s, p.sign, V, r,
                                       xt, zp, hs);
        if (e != hipSuccess) return hip_fail(e, "scalar-LUT pre-pass (T <= 8)");
        Lut8Args q;
        memset(&q, 0, sizeof q);
        q.codes = reinterpret_cast<const uint32_t*>(base + L.codes_off);
        q.lut = reinterpret_cast<const uint16_t*>(base + L.cb_off);
        q.sc = reinterpret_cast<const uint16_t*>(base + L.sc_off);
        q.x = xt;
        q.y = static_cast<uint16_t*>(y);
        q.U = U;
        q.zp = zp;
        q.nch = lut8_planes(K, hb);
        q.bits = bits;
        q.N = N;
        q.K = K;
        q.T = T;
        q.r = r;
        e = launch_lut8(q, hs);
        if (e != hipSuccess) return hip_fail(e, "scalar-LUT projection (T <= 8)");
        return ok();
    }
    // x~ = R(x . s): the rotation kernel with a 1-wide block is the plain scale and sign
    hipError_t e = launch_rotate(T, K, hb, x, 0, p.s, p.sign, xt, 1, hs);
    if (e != hipSuccess) return hip_fail(e, "rotate (mixer input)");
    if (r > 0) {
        // z = x~ V^T has few outputs: split K over the CUs, then sum the planes
        GemmArgs g;
        memset(&g, 0, sizeof g);
        g.kind = kGemmDense32;
        g.N = r;
        g.K = K;
        g.T = T;
        g.x = xt;
        g.dense = V;
        g.ksplit = gemm_split(kGemmDense32, r, K, T, kLutSplitCUs);
        float* zp = reinterpret_cast<float*>(wb + align256(size_t(T) * K * 2) +
                                             align256(size_t(T) * r * 4));
        g.out32 = g.ksplit > 1 ? zp : z;
        e = launch_gemm(g, hs);
        if (e != hipSuccess) return hip_fail(e, "rank-r projection");
        if (g.ksplit > 1) {
            e = launch_split_sum(T * r, g.ksplit, zp, z, hs);
            if (e != hipSuccess) return hip_fail(e, "rank-r projection (K split sum)");
        }
    }
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.kind = bits == 2 ? kGemmLUT2 : kGemmLUT4;
    g.N = N;
    g.K = K;
    g.T = T;
    g.x = xt;
    g.codes[0] = base + L.codes_off;
    g.cb[0] = reinterpret_cast<const uint32_t*>(base + L.cb_off);
    g.sc[0] = reinterpret_cast<const uint16_t*>(base + L.sc_off);
    g.z = z;
    g.U = U;
    g.r = r;
    g.out16 = static_cast<uint16_t*>(y);
    // too few row tiles to fill the CUs: split K into scaled FP32 planes, then sum them
    const int ls = gemm_split(g.kind, N, K, T, kLutSplitCUs);
    if (trace_on())
        trace("scalar-LUT %d-bit N=%d K=%d T=%d r=%d: rotation; %s; %s LUT product%s", bits, N,
              K, T, r, r > 0 ? "rank-r product z = V x~ (K split, sum)" : "no rank term",
              T >= kVq3mmMinT ? "register-decode" : "tiled",
              ls > 1 ? " K-split + reduction" : "");
    if (ls > 1) {
        const int zs = gemm_split(kGemmDense32, r ? r : 1, K, T, kLutSplitCUs);
        float* lp = reinterpret_cast<float*>(wb + align256(size_t(T) * K * 2) +
                                             align256(size_t(T) * (r ? r : 1) * 4) +
                                             (zs > 1 ? align256(size_t(zs) * T * (r ? r : 1) * 4) : 0));
        g.ksplit = ls;
        g.out32 = lp;
        e = launch_gemm(g, hs);
        if (e != hipSuccess) return hip_fail(e, "scalar-LUT projection (K split)");
        e = launch_split_reduce(T, N, ls, lp, nullptr, static_cast<uint16_t*>(y), hs);
        if (e != hipSuccess) return hip_fail(e, "scalar-LUT projection (K split sum)");
        return ok();
    }
    e = launch_gemm(g, hs);
    if (e != hipSuccess) return hip_fail(e, "scalar-LUT projection");
    return ok();
}


}  // namespace

extern "C" {

vqmlp_status vqmlp_lut_forward(int bits, int N, int K, int T, const void* packed,
                               const uint16_t* U, const uint16_t* V, int r, const uint16_t* s,
                               const int8_t* sign, int had_block, const void* x, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_forward: T=%d", T);
    vqmlp_status st = lut_args(bits, N, K, r, had_block);
    if (st) return st;
    if (T == 0) return ok();
    vqmlp_lut_plan p;
    st = lut_validate(bits, N, K, packed, U, V, r, s, sign, had_block, &p);
    if (st) return st;
    return lut_run(p, T, x, y, workspace, workspace_bytes, stream);
}

vqmlp_status vqmlp_lut_create(int bits, int N, int K, const void* packed, const uint16_t* U,
                              const uint16_t* V, int r, const uint16_t* s, const int8_t* sign,
                              int had_block, vqmlp_lut_plan** out) {
    if (!out) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_create: null pointer");
    *out = nullptr;
    vqmlp_lut_plan tmp;
    vqmlp_status st = lut_validate(bits, N, K, packed, U, V, r, s, sign, had_block, &tmp);
    if (st) return st;
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        tmp.cus = std::min(cus, kArgmaxMaxGroups);
    }
    vqmlp_lut_plan* p = new (std::nothrow) vqmlp_lut_plan(tmp);
    if (!p) return fail(VQMLP_ERR_INVALID_ARG, "out of host memory");
    *out = p;
    return ok();
}

vqmlp_status vqmlp_lut_destroy(vqmlp_lut_plan* plan) {
    delete plan;
    return ok();
}

vqmlp_status vqmlp_lut_plan_forward(const vqmlp_lut_plan* plan, int T, const void* x, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_plan_forward: null plan");
    return lut_run(*plan, T, x, y, workspace, workspace_bytes, stream);
}

vqmlp_status vqmlp_lut_plan_argmax(const vqmlp_lut_plan* plan, int T, const void* x,
                                   int32_t* index, float* value, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!plan) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_plan_argmax: null plan");
    const vqmlp_lut_plan& p = *plan;
    const int N = p.N, K = p.K;
    if (T < 0 || T > kSkinnyT)
        return fail(VQMLP_ERR_UNSUPPORTED, "the argmax head takes T <= %d (T=%d)", kSkinnyT, T);
    if (T == 0) return ok();
    if (p.r != 0) return fail(VQMLP_ERR_UNSUPPORTED, "the argmax head takes no low-rank factors");
    const int hb = p.had_block ? p.had_block : 1;
    if (K > kLut8MaxK || lut8_chunk(K, hb) < 64 || !aligned(p.s, 16) || !aligned(p.sign, 8))
        return fail(VQMLP_ERR_UNSUPPORTED,
                    "the argmax head takes K <= %d, power-of-two column chunks, s 16- and sign "
                    "8-byte aligned (K=%d)", kLut8MaxK, K);
    if (!x || !index || !workspace)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_lut_plan_argmax: null pointer");
    if (!aligned(x, 16) || !aligned(workspace, 256) || !aligned(index, 4) || !aligned(value, 4))
        return fail(VQMLP_ERR_INVALID_ARG, "x must be 16-byte aligned, the workspace 256");
    size_t need = 0;
    vqmlp_lut_workspace_bytes(N, K, T, 0, &need);
    if (workspace_bytes < need)
        return fail(VQMLP_ERR_WORKSPACE, "workspace holds %zu bytes, this call needs %zu",
                    workspace_bytes, need);
    uint8_t* wb = static_cast<uint8_t*>(workspace) + 256;
    uint16_t* xt = reinterpret_cast<uint16_t*>(wb);
    float* pval = reinterpret_cast<float*>(wb + align256(size_t(T) * K * 2));
    int* pidx = reinterpret_cast<int*>(pval + kArgmaxMaxGroups * kSkinnyT);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (trace_on())
        trace("argmax head %d-bit N=%d K=%d T=%d: pre-pass (rotation); persistent head "
              "(%d workgroups); candidate merge", p.bits, N, K, T, lut8_argmax_grid(N, p.cus));
    hipError_t e = launch_lut8_pre(T, K, hb, static_cast<const uint16_t*>(x), p.s, p.sign, nullptr, 0,
                                   xt, nullptr, hs);
    if (e != hipSuccess) return hip_fail(e, "argmax head: input scale and rotation");
    Lut8Args q;
    memset(&q, 0, sizeof q);
    q.codes = reinterpret_cast<const uint32_t*>(p.base + p.L.codes_off);
    q.lut = reinterpret_cast<const uint16_t*>(p.base + p.L.cb_off);
    q.sc = reinterpret_cast<const uint16_t*>(p.base + p.L.sc_off);
    q.x = xt;
    q.bits = p.bits;
    q.N = N;
    q.K = K;
    q.T = T;
    e = launch_lut8_argmax(q, p.cus, pval, pidx, index, value, hs);
    if (e != hipSuccess) return hip_fail(e, "argmax head");
    return ok();
}

}  // extern "C"

// ==================================================================== 2x16 vector LUT
namespace {

constexpr uint32_t kKindVq2 = 216;  // packed-header kind of the 2x16 format (16 entries)

vqmlp_status vq2_shape(int N, int K) {
    if (N <= 0 || K <= 0 || N > (1 << 20) || K > (1 << 20) || N % 32 || K % 32)
        return fail(VQMLP_ERR_INVALID_ARG, "2x16 matrix %dx%d: both must be multiples of 32", N, K);
    return VQMLP_OK;
}

Layout vq2_layout(int N, int K) {
    Layout L;
    L.codes_off = kHeaderBytes;
    L.codes_bytes = size_t(N / 2) * K / 2;  // 4 bits per code, [N/2][K/8] words
    L.cb_off = align256(L.codes_off + L.codes_bytes);
    L.cb_bytes = size_t(N / 8) * 16 * 4;
    L.sc_off = align256(L.cb_off + L.cb_bytes);
    L.sc_bytes = size_t(N) * 2;
    L.total = align256(L.sc_off + L.sc_bytes);
    return L;
}

// Validate one packed 2x16 matrix (header read through a synchronous copy) and view it.
vqmlp_status vq2_view_checked(const void* dev, int N, int K, const char* name, VQ3View* v) {
    vqmlp_status st = vq2_shape(N, K);
    if (st) return st;
    const Layout L = vq2_layout(N, K);
    PackedHeader h;
    if ((st = read_device_header(dev, &h, name))) return st;
    if ((st = check_header(h, N, K, kKindVq2, 16, L, name))) return st;
    const uint8_t* base = static_cast<const uint8_t*>(dev);
    v->codes = base + L.codes_off;
    v->cb = reinterpret_cast<const uint32_t*>(base + L.cb_off);
    v->sc = reinterpret_cast<const uint16_t*>(base + L.sc_off);
    v->N = N;
    v->K = K;
    return VQMLP_OK;
}

}  // namespace

struct vqmlp_vq2_plan {
    int N, K;
    const uint8_t* base;
    Layout L;
};

extern "C" {

vqmlp_status vqmlp_vq2_packed_bytes(int N, int K, size_t* bytes) {
    if (!bytes) return fail(VQMLP_ERR_INVALID_ARG, "bytes is NULL");
    vqmlp_status st = vq2_shape(N, K);
    if (st) return st;
    *bytes = vq2_layout(N, K).total;
    return ok();
}

vqmlp_status vqmlp_vq2_pack(int N, int K, const uint8_t* codes, const uint16_t* codebook,
                            const uint16_t* row_scale, void* packed, size_t bytes) {
    vqmlp_status st = vq2_shape(N, K);
    if (st) return st;
    if (!codes || !codebook || !row_scale || !packed)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_pack: null pointer");
    const Layout L = vq2_layout(N, K);
    if (bytes < L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_pack: buffer holds %zu bytes, needs %zu",
                    bytes, L.total);
    const size_t nc = size_t(N / 2) * K;
    for (size_t i = 0; i < nc; ++i)
        if (codes[i] > 15)
            return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_pack: code %u > 15 at %zu", codes[i], i);
    uint8_t* out = static_cast<uint8_t*>(packed);
    memset(out, 0, L.total);
    PackedHeader h = header_of(N, K, kKindVq2, 16, L);
    memcpy(out, &h, sizeof h);
    uint32_t* words = reinterpret_cast<uint32_t*>(out + L.codes_off);
    for (size_t i = 0; i < nc; ++i) words[i / 8] |= uint32_t(codes[i]) << (4 * (i % 8));
    memcpy(out + L.cb_off, codebook, L.cb_bytes);
    memcpy(out + L.sc_off, row_scale, L.sc_bytes);
    return ok();
}

vqmlp_status vqmlp_vq2_unpack(int N, int K, const void* packed, size_t bytes, uint8_t* codes,
                              uint16_t* codebook, uint16_t* row_scale) {
    vqmlp_status st = vq2_shape(N, K);
    if (st) return st;
    if (!packed || !codes || !codebook || !row_scale)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_unpack: null pointer");
    const Layout L = vq2_layout(N, K);
    if (bytes < L.total)
        return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_unpack: buffer holds %zu bytes, needs %zu",
                    bytes, L.total);
    const uint8_t* in = static_cast<const uint8_t*>(packed);
    PackedHeader h;
    memcpy(&h, in, sizeof h);
    if ((st = check_header(h, N, K, kKindVq2, 16, L, "vqmlp_vq2_unpack"))) return st;
    const uint32_t* words = reinterpret_cast<const uint32_t*>(in + L.codes_off);
    const size_t nc = size_t(N / 2) * K;
    for (size_t i = 0; i < nc; ++i) codes[i] = uint8_t((words[i / 8] >> (4 * (i % 8))) & 15u);
    memcpy(codebook, in + L.cb_off, L.cb_bytes);
    memcpy(row_scale, in + L.sc_off, L.sc_bytes);
    return ok();
}

vqmlp_status vqmlp_vq2_create(int N, int K, const void* packed, vqmlp_vq2_plan** out) {
    if (!out) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_create: null pointer");
    *out = nullptr;
    vqmlp_status st = vq2_shape(N, K);
    if (st) return st;
    if (K > kVq2MaxK)
        return fail(VQMLP_ERR_UNSUPPORTED, "2x16 projection: K=%d above %d", K, kVq2MaxK);
    if (!packed) return fail(VQMLP_ERR_INVALID_ARG, "2x16 projection: null packed buffer");
    if ((st = check_device())) return st;
    const Layout L = vq2_layout(N, K);
    PackedHeader h;
    if ((st = read_device_header(packed, &h, "vq2"))) return st;
    if ((st = check_header(h, N, K, kKindVq2, 16, L, "vq2"))) return st;
    vqmlp_vq2_plan* p = new (std::nothrow) vqmlp_vq2_plan{N, K, static_cast<const uint8_t*>(packed), L};
    if (!p) return fail(VQMLP_ERR_INVALID_ARG, "out of host memory");
    *out = p;
    return ok();
}

vqmlp_status vqmlp_create_vq2(const vqmlp_desc* desc, vqmlp_plan** out) {
    return create_plan(desc, out, true, vq2_view_checked);
}

vqmlp_status vqmlp_vq2_destroy(vqmlp_vq2_plan* plan) {
    delete plan;
    return ok();
}

vqmlp_status vqmlp_vq2_plan_forward(const vqmlp_vq2_plan* plan, int T, const void* x, void* y,
                                    void* stream) {
    if (!plan) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_plan_forward: null plan");
    if (T < 0 || T > kSkinnyT)
        return fail(VQMLP_ERR_UNSUPPORTED, "the 2x16 projection takes T <= %d (T=%d)", kSkinnyT, T);
    if (T == 0) return ok();
    if (!x || !y) return fail(VQMLP_ERR_INVALID_ARG, "vqmlp_vq2_plan_forward: null x or y");
    if (!aligned(x, 16)) return fail(VQMLP_ERR_INVALID_ARG, "x must be 16-byte aligned");
    const vqmlp_vq2_plan& p = *plan;
    Vq2Args a;
    memset(&a, 0, sizeof a);  // one matrix (no second codes)
    a.codes = reinterpret_cast<const uint32_t*>(p.base + p.L.codes_off);
    a.cb = reinterpret_cast<const uint32_t*>(p.base + p.L.cb_off);
    a.sc = reinterpret_cast<const uint16_t*>(p.base + p.L.sc_off);
    a.x = static_cast<const uint16_t*>(x);
    a.y = static_cast<uint16_t*>(y);
    a.out32 = nullptr;
    a.N = p.N;
    a.K = p.K;
    a.T = T;
    a.ldk = p.K;
    a.nsplit = 1;
    a.o32_t = a.o32_s = 0;
    if (trace_on()) trace("2x16 projection N=%d K=%d T=%d: projection kernel", p.N, p.K, T);
    const hipError_t e = launch_vq2_8(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "2x16 projection");
    return ok();
}

}  // extern "C"
