// 2x16 vector-LUT projection at T <= 8 tokens: y[t][r] = sc[r] * sum_j cb[r/8][code[r/2][j]][r%2] x[t][j]
// (the two-bit vector LUT of the model card's previous packages, section "Release 0.2",
// format table: 16 two-component centroids per group of 8 output rows, one four-bit index per
// pair of output channels, per-channel scales).
//
// Workgroup: one tile of 16 row pairs (32 output rows) x 16 K slices, one wave per slice.  Lane
// (pair i = l mod 16, group g = l / 16) of a wave streams one contiguous run of code words (8
// codes per word, code j at bits 4 (j mod 8) of word j / 8 of its pair row), g taking a quarter
// of the slice.  A code is looked up in LDS as the half2 (component 0, component 1) of its
// centroid, which is the A operand of v_mfma_f32_16x16x32_f16 when the contraction index is
// (column, component): A[i][(j, c)] = cb[code[i][j]][c].  The token operand then carries the
// component as well: B[(j, c)][n] = x[n mod 8][j] if c == n / 8, else 0, so output column n
// holds row 2 i + n / 8 of token n mod 8, and all 16 columns are used.
#include "device.h"
#include "internal.h"

namespace vqmlp {
namespace {

constexpr int kVW = 16;                    // waves: 16 K slices
constexpr int kVMaxK = kVq2MaxK;           // x rows staged in LDS
constexpr int kVXRow = kVMaxK + 8;         // LDS row of x in halves (padded against bank conflicts)
constexpr int kVMaxU = (kVMaxK / 32 + kVW - 1) / kVW;  // units (32 columns, one word per lane) per slice
constexpr int kVRunV = (kVMaxU + 3) / 4;   // 16-byte loads per lane
constexpr int kVTab = 16 * 32;             // 16 centroids x 32 bank columns
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));

// LDS byte address of the centroid that bits sh..sh+3 of d select, in table column lb
__device__ __forceinline__ uint32_t vq2_addr(uint32_t d, uint32_t sh, uint32_t lb) {
    uint32_t a;
    asm("v_bfe_u32 %0, %1, %2, 4\n\tv_lshl_or_b32 %0, %0, 7, %3" : "=&v"(a) : "v"(d), "s"(sh), "v"(lb));
    return a;
}

}  // namespace

// Persistent: workgroup b takes the tiles b, b + G, ... of its (matrix, K slice) grid row; x is
// staged once, and while a tile's lookups run, the next tile's code runs, centroid words and row
// scales are already in flight (centroid tables and partial sums double-buffered in LDS, one
// barrier per tile: a tile's epilogue runs beside the next tile's products).
__global__ void __launch_bounds__(kVW * 64, 1) k_vq2_8(Vq2Args a) {
    constexpr int kOffX = 2 * kVTab * 4, kOffRed = kOffX + kSkinnyT * kVXRow * 2;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kOffRed + 2 * kVW * 64 * 16];
    auto& tab = *reinterpret_cast<uint32_t (*)[2][kVTab]>(lds);
    auto& xs = *reinterpret_cast<uint16_t (*)[kSkinnyT][kVXRow]>(lds + kOffX);
    auto& red = *reinterpret_cast<f32x4 (*)[2][kVW][64]>(lds + kOffRed);  // [buffer][wave][lane]

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, T = a.T, N = a.N, ntile = a.N / 32, G = gridDim.x;
    // grid row: matrix mat (the second one when a.codes2 is set), K slice sl
    const int mat = int(blockIdx.y) / a.nsplit, sl = int(blockIdx.y) % a.nsplit;
    const uint32_t* const mcodes = mat ? a.codes2 : a.codes;
    const uint32_t* const mcb = mat ? a.cb2 : a.cb;
    const uint16_t* const msc = mat ? a.sc2 : a.sc;
    const int ldk = a.ldk, k0 = sl * K;  // this workgroup's K slice
    const int nu = K / 32, u0 = w * nu / kVW, nus = (w + 1) * nu / kVW - u0;

    // lane (pair i, group g): kVRunV 16-byte loads of its code run whatever nus is; words past
    // the run are unused and past the last pair row they fall in the codebook section
    const int i = l & 15, g = l >> 4;
    auto load_codes = [&](int b, uint32_t (&c)[kVRunV * 4]) {
        const uint32_t* crun = mcodes + size_t(b * 16 + i) * (ldk / 8) + k0 / 8 + u0 * 4 + g * nus;
#pragma unroll
        for (int v = 0; v < kVRunV; ++v) {
            const u32x4a q = *reinterpret_cast<const u32x4a*>(crun + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) c[4 * v + e] = q[e];
        }
    };
    // centroid words: thread (entry te, bank column tc), column tc serving pair row tc mod 16
    // (a group of 4 pairs = 8 output rows); stored by threads below kVTab
    const int te = (tid >> 5) & 15, tc = tid & 31;
    auto load_tw = [&](int b) { return mcb[size_t((b * 16 + (tc & 15)) >> 2) * 16 + te]; };
    // epilogue thread (pair ei, column en): every thread loads a scale (past 256 a duplicate), so
    // no load sits under a branch
    const int ei = (tid >> 4) & 15, en = tid & 15;
    auto load_sc = [&](int b) { return msc[2 * (b * 16 + ei) + (en >> 3)]; };

    int blk = blockIdx.x;
    uint32_t tw = load_tw(blk);
    uint16_t esc = load_sc(blk);
    uint32_t cw[kVRunV * 4];
    load_codes(blk, cw);
    // x rows (past T zero), all loads before the stores
    constexpr int kXPer = kSkinnyT * kVMaxK / 8 / (kVW * 64);
    const int c8n = K / 8;
    {
        u32x4 xv[kXPer];
#pragma unroll
        for (int k = 0; k < kXPer; ++k) {
            // no branch around the load (a load under a divergent branch is waited for inside
            // it, and that wait covers every older load): a valid address, zeroed if unused
            const int q = tid + k * kVW * 64, t = q / c8n, c8 = (q % c8n) * 8;
            const bool on = q < kSkinnyT * c8n && t < T;
            xv[k] = *reinterpret_cast<const u32x4*>(a.x + (on ? size_t(t) * ldk + k0 + c8 : 0));
            if (!on) xv[k] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kXPer; ++k) {
            const int q = tid + k * kVW * 64, t = q / c8n, c8 = (q % c8n) * 8;
            if (q < kSkinnyT * c8n) *reinterpret_cast<u32x4*>(&xs[t][c8]) = xv[k];
        }
    }

    // Lane column n: token n mod 8, component n / 8; its B word for column j keeps x in the half
    // of its component and zero in the other (v_perm byte selectors: 4..7 pick the source word,
    // 12 gives zero)
    const char* tb0 = reinterpret_cast<const char*>(&tab[0][0]);
    const int n = l & 15, tok = n & 7;
    const uint32_t selE = n < 8 ? 0x0C0C0504u : 0x05040C0Cu;  // low half of the word
    const uint32_t selO = n < 8 ? 0x0C0C0706u : 0x07060C0Cu;  // high half
    // output (pair ei, column en) of tile pblk from partials buffer pb: register ei mod 4 of lane
    // 16 (ei / 4) + en; the 16 slices summed in order, scaled in FP32, rounded once
    auto finish = [&](int pb, int pblk, uint16_t pesc) {
        if (tid < 256) {
            const int el = 16 * (ei >> 2) + en, eq = ei & 3;
            float v = 0.f;
#pragma unroll
            for (int s = 0; s < kVW; ++s) v += red[pb][s][el][eq];
            const int t = en & 7, row = 2 * (pblk * 16 + ei) + (en >> 3);
            if (t < T) {
                if (a.out32)
                    a.out32[size_t(mat) * a.o32_m + size_t(sl) * a.o32_s + size_t(t) * a.o32_t + row] = v;
                else
                    a.y[size_t(t) * N + row] = uint16_t(f2h(v * h2f(pesc)));
            }
        }
    };
    // The partials alternate between two buffers, so one barrier per tile suffices: a tile's
    // epilogue runs after the next tile's barrier, beside that tile's products.
    int pblk = -1, ppar = 0;
    uint16_t pesc = 0;
    for (int it = 0; blk < ntile; ++it, blk += G) {
        const int par = it & 1;
        if (tid < kVTab) tab[par][te * 32 + tc] = tw;
        // the next tile's words, requested now (none after the workgroup's last tile)
        const bool more = blk + G < ntile;  // uniform
        uint32_t twn = 0, cn[kVRunV * 4];
        uint16_t escn = 0;
        if (more) {
            twn = load_tw(blk + G);
            escn = load_sc(blk + G);
            load_codes(blk + G, cn);
        }
        // this tile's table (and x) written; the last tile's partials complete, and those of the
        // tile before it (this buffer) consumed
        __syncthreads();
        if (pblk >= 0) finish(ppar, pblk, pesc);
        const uint32_t lb = (uint32_t(l & 31) << 2) | uint32_t(par * kVTab * 4);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kVMaxU; ++u) {
            if (u < nus) {  // uniform
                const int jb = 32 * u0 + 8 * (g * nus + u);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    u32x4 A, B;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        A[p] = *reinterpret_cast<const uint32_t*>(tb0 + vq2_addr(cw[u], 16 * s + 4 * p, lb));
                    const u32x2 xw = *reinterpret_cast<const u32x2*>(&xs[tok][jb + 4 * s]);
                    B[0] = __builtin_amdgcn_perm(xw[0], 0u, selE);
                    B[1] = __builtin_amdgcn_perm(xw[0], 0u, selO);
                    B[2] = __builtin_amdgcn_perm(xw[1], 0u, selE);
                    B[3] = __builtin_amdgcn_perm(xw[1], 0u, selO);
                    acc = mfma16x16x32(A, B, acc);
                }
            }
        }
        red[par][w][l] = acc;
        pblk = blk;
        ppar = par;
        pesc = esc;
        if (more) {
#pragma unroll
            for (int k = 0; k < kVRunV * 4; ++k) cw[k] = cn[k];
            tw = twn;
            esc = escn;
        }
    }
    __syncthreads();
    if (pblk >= 0) finish(ppar, pblk, pesc);
}

namespace {
// compute units of the current device (cached per device; workgroups of the persistent grid)
int vq2_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
            c = 256;
        cache[dev] = c;
    }
    return cache[dev];
}
}  // namespace

hipError_t launch_vq2_8(const Vq2Args& a, hipStream_t st) {
    if (!a.codes || !a.cb || !a.sc || !a.x || !(a.y || a.out32) || a.N < 32 || a.N % 32 ||
        a.K < 32 || a.K % 32 || a.K > kVMaxK || a.T < 1 || a.T > kSkinnyT || a.nsplit < 1 ||
        a.ldk != a.K * a.nsplit || (a.nsplit > 1 && !a.out32) ||
        (a.codes2 && (!a.cb2 || !a.sc2 || !a.out32)))
        return hipErrorInvalidValue;
    const int ntile = a.N / 32, cus = vq2_cus(), rows = a.nsplit * (a.codes2 ? 2 : 1);
    // persistent over the row tiles of each (matrix, slice): about one workgroup per CU in all
    const int per = (cus + rows - 1) / rows;
    const int G = ntile < per ? ntile : per;
    hipLaunchKernelGGL(k_vq2_8, dim3(G, rows), dim3(kVW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace vqmlp
