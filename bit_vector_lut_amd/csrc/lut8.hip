// lut8.hip -- scalar-LUT projection for T <= 8 rows (token mixers at decode size), gfx950.
//
// Format (model card "anemll/anemll-forge-qwen3.8-27B", format table, "Token mixers" row): 2- or
// 4-bit codes, one table of 2^bits binary16 scalars per 8 output rows, a binary16 scale per row,
// rank-r binary16 factors U [N][r], V [r][K]:  y = sc . (W_lut x~) + U z,  z = V x~.
//
// At T <= 8 the projection streams each code once and multiplies it by at most 8 tokens, so the
// layout is chosen for the code stream: a workgroup of 16 waves owns 32 output rows (two 16-row
// tiles) and splits K in 8 slices; every lane issues all of its code loads (one 32-bit word per
// 64-column unit for 2-bit codes, two for 4-bit) before anything else, x~ (at most 8 x 5120
// binary16) is staged once per workgroup in LDS, and the 16 waves' partial sums meet in LDS.
//
// Product: v_mfma_f32_16x16x32_f16 with A = the decoded weights of 16 rows and B = x~ (column n =
// token n mod 8; columns 8..15 repeat tokens 0..7 and their outputs are never read).  A wave's K slice of nus 64-column units is cut into four runs of
// 16 nus columns, one per lane group g = l / 16; MFMA step (u, s) takes columns 16 u + 8 s + 0 .. 7
// of each group's run in both operands, so a lane's codes for the whole slice are one contiguous
// run of 16 nus codes in the row-major packing (nus or 2 nus consecutive words).  Lookups go to tables replicated over the 32 bank
// columns (column c serves the lanes with l % 32 == c, whose row lies in group (c % 16) / 8):
// 2-bit codes are looked up in pairs (16 entries, each the two binary16 weights of a code pair,
// so the 32-bit read is the operand word), 4-bit codes one by one (16 entries, 16-bit reads).
//
// The output head (k_lut8_argmax) runs the same product persistently over 32-row blocks and keeps a
// running per-token argmax instead of writing logits.
#include "device.h"
#include "internal.h"

namespace vqmlp {

namespace {
constexpr int kW = 16;                  // waves per workgroup: 2 row tiles x 8 K slices
constexpr int kKS = 8;                  // K slices
constexpr int kMaxK = kLut8MaxK;        // x~ rows staged in LDS
constexpr int kXRow = kMaxK + 8;        // LDS row of x~ in halves (padded against bank conflicts)
constexpr int kMaxU = (kMaxK / 64 + kKS - 1) / kKS;  // units per slice
constexpr int kTabDw = 16 * 32;         // one table: 16 entries x 32 bank columns

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
// The value of lane l ^ D (D a power of two below 64) in lane l of a wave: row-local DPP moves for
// 1 (quad_perm [1,0,3,2]), 2 (quad_perm [2,3,0,1]) and 8 (row_ror:8, which is xor 8 inside a row
// of 16), a swizzle inside each half-wave for 4 and 16 (bit-mask mode: xor mask D, and mask 0x1F),
// a backward permute across the halves for 32.
template <int D>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(D > 0 && D < 64 && (D & (D - 1)) == 0, "lane distance");
    const int i = __builtin_bit_cast(int, v);
    int r;
    if constexpr (D == 1)
        r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);
    else if constexpr (D == 2)
        r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);
    else if constexpr (D == 8)
        r = __builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, false);
    else if constexpr (D == 4 || D == 16)
        r = __builtin_amdgcn_ds_swizzle(i, (D << 10) | 0x1F);
    else
        r = __builtin_amdgcn_ds_bpermute(int(((threadIdx.x & 63) ^ D) << 2), i);
    return __builtin_bit_cast(float, r);
}

// The table words of two 4-bit codes (bits sh..sh+3 and sh+4..sh+7 of d) as one binary16 pair:
// two 16-bit LDS reads joined by one byte permute (two field extracts, two address merges).
// LDS byte address of the entry that bits sh..sh+3 of d select, in the table column lb: a field
// extract and a shift-or (the compiler would otherwise emit shift, mask and add).
__device__ __forceinline__ uint32_t lut_addr(uint32_t d, uint32_t sh, uint32_t lb) {
    uint32_t a;
    asm("v_bfe_u32 %0, %1, %2, 4\n\tv_lshl_or_b32 %0, %0, 7, %3" : "=&v"(a) : "v"(d), "s"(sh), "v"(lb));
    return a;
}
__device__ __forceinline__ uint32_t look_pair4(const char* tb, uint32_t lb, uint32_t d, int sh) {
    h2v v;
    v.x = *reinterpret_cast<const _Float16*>(tb + lut_addr(d, sh, lb));
    v.y = *reinterpret_cast<const _Float16*>(tb + lut_addr(d, sh + 4, lb));
    return __builtin_bit_cast(uint32_t, v);
}
// the half2 table word of the 2-bit code pair in bits sh..sh+3 of d
__device__ __forceinline__ uint32_t look_pair2(const char* tb, uint32_t lb, uint32_t d, int sh) {
    return *reinterpret_cast<const uint32_t*>(tb + lut_addr(d, sh, lb));
}
// A wave's products over its K slice: nus units of 64 columns, two matrix-core steps each, on the
// lane's code run cw.  A = the decoded weights of the wave's 16 rows, B = x~ (column n = token n mod 8;
// columns 8..15 repeat tokens 0..7 and their outputs are never read, so no masking).  FULL: the
// slice has all kMaxU units, and the loop runs without a check per unit, so that the scheduler can
// move a unit's lookups ahead of the previous unit's waits.
template <int BITS, bool FULL, int NW>
__device__ __forceinline__ f32x4 lut_products(const uint32_t (&cw)[NW], int nus, int u0, int g,
                                              const char* tb, uint32_t lb,
                                              const uint16_t (&xs)[kSkinnyT][kXRow], int n) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMaxU; ++u) {
        if (FULL || u < nus) {  // uniform
            const int kb = u0 * 64 + 16 * (g * nus + u);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 A;
                if constexpr (BITS == 2) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) A[p] = look_pair2(tb, lb, cw[u], 16 * s + 4 * p);
                } else {
                    const uint32_t d = cw[2 * u + s];
#pragma unroll
                    for (int p = 0; p < 4; ++p) A[p] = look_pair4(tb, lb, d, 8 * p);
                }
                const u32x4 B = *reinterpret_cast<const u32x4*>(&xs[n & (kSkinnyT - 1)][kb + 8 * s]);
                acc = mfma16x16x32(A, B, acc);
            }
        }
    }
    return acc;
}
constexpr int kMaxR = 256;              // rank of the low-rank term
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));  // 4-byte aligned
}  // namespace

// FULL: K = kMaxK, so that every wave's K slice holds all kMaxU units (the products then run
// without a check per unit; chosen at launch)
template <int BITS, bool FULL>
__global__ void __launch_bounds__(kW * 64, 1) k_lut8(Lut8Args a) {
    constexpr int CW = BITS == 2 ? 1 : 2;  // code words per lane and unit
    // one LDS block with the tables at address 0 (a lookup address is the entry and lane bits)
    constexpr int kOffX = 2 * kTabDw * 4, kOffRed = kOffX + kSkinnyT * kXRow * 2;
    constexpr int kOffZ = kOffRed + kW * 64 * 16, kOffZP = kOffZ + kSkinnyT * kMaxR * 4;
    constexpr int kOffU = kOffZP + kSkinnyT * kMaxR * 4;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kOffU + 32 * kMaxR * 2];
    auto& tab = *reinterpret_cast<uint32_t (*)[2][kTabDw]>(lds);
    auto& xs = *reinterpret_cast<uint16_t (*)[kSkinnyT][kXRow]>(lds + kOffX);
    auto& red = *reinterpret_cast<f32x4 (*)[kW][64]>(lds + kOffRed);
    float* zs = reinterpret_cast<float*>(lds + kOffZ);    // z [8][r] (rows past T zero)
    float* zpart = reinterpret_cast<float*>(lds + kOffZP);  // partial sums of z by plane class
    uint16_t* us = reinterpret_cast<uint16_t*>(lds + kOffU);  // U rows of the workgroup [32][r]

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, T = a.T, N = a.N;
    const int row0 = blockIdx.x * 32;
    const int rt = w / kKS, ks = w % kKS;  // row tile, K slice (uniform)
    const int nu = K / 64, u0 = ks * nu / kKS, nus = (ks + 1) * nu / kKS - u0;

    // ---- the code stream first: lane (row i, column group g) of its row tile
    const int i = l & 15, g = l >> 4;
    // The lane's run is kMaxU * CW words read as 16-byte loads whatever nus is: words past the
    // run are never used, and past the last row they fall in the table section that follows
    // the codes in the packed buffer.
    const uint32_t* crun = a.codes + size_t(row0 + rt * 16 + i) * (K * BITS / 32) +
                           u0 * (64 * BITS / 32) + g * nus * (16 * BITS / 32);
    constexpr int kRunW = kMaxU * CW, kRunV = (kRunW + 3) / 4;
    uint32_t cw[kRunV * 4];
#pragma unroll
    for (int v = 0; v < kRunV; ++v) {
        const u32x4a q = *reinterpret_cast<const u32x4a*>(crun + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) cw[4 * v + e] = q[e];
    }

    // ---- the epilogue's U rows, requested now: the workgroup's 32 rows are one contiguous block
    // of 32 r binary16, one 16-byte chunk per thread (threads 0 .. 255 own one output each)
    const int ert = tid >> 7, ej = tid & 127, ell = ej >> 2, eq = ej & 3;
    const int el = (ell >> 3) * 16 + (ell & 7);  // lanes holding tokens 0 .. 7
    const int erow = row0 + ert * 16 + 4 * (el >> 4) + eq;
    // Loads are issued without a branch around them (clamped to a valid address where the value
    // is not needed): a load under a divergent branch has its value used inside the branch, and
    // that wait would cover every load issued before it.
    const uint16_t escb = a.sc[tid < 256 ? erow : row0];
    const int nuc = 4 * a.r;  // 16-byte chunks of the 32 U rows
    u32x4 uv = u32x4{0u, 0u, 0u, 0u};
    if (a.r > 0)  // uniform
        uv = *reinterpret_cast<const u32x4*>(a.U + size_t(row0) * a.r + 8 * (tid < nuc ? tid : 0));

    // ---- every other global load before the first LDS store (a store that needs a loaded value
    // waits for every older load, so one round trip covers them all): table entries (thread: row
    // tile, entry e, bank column c), z, x~
    const int trt = tid >> 9, te = (tid >> 5) & 15, tc = tid & 31;
    const int grp = (row0 + trt * 16) / 8 + ((tc & 15) >> 3);
    const uint32_t t0 = a.lut[BITS == 2 ? grp * 4 + (te & 3) : grp * 16 + te];
    const uint32_t t1 = BITS == 2 ? a.lut[grp * 4 + (te >> 2)] : 0u;
    // z = the sum of the pre-pass planes: ZG threads share an entry q, thread class p summing the
    // planes p, p + ZG, ... in order; the classes are summed in order after the barrier (entries
    // of tokens past T are zero).  The first kZL planes of the first entry are requested here and
    // summed after the x~ loads are issued; more planes or a second entry (E > 1024) follow.
    const int E = kSkinnyT * a.r, ZG = E == 0 || E >= kW * 64 ? 1 : (kW * 64) / E;
    constexpr int kZL = 16;
    auto zentry = [&](int k, int& q, int& p) -> bool {
        q = ZG > 1 ? tid % E : tid + k * kW * 64;
        p = ZG > 1 ? tid / E : 0;
        return (k == 0 || ZG == 1) && p < ZG && q < E && q / a.r < T;
    };
    // (with r == 0 the first batch reads the codes instead, a valid address, and is discarded)
    const float* zsrc = a.r > 0 ? a.zp : reinterpret_cast<const float*>(a.codes);
    auto zload = [&](float (&zq)[kZL], int c0, int q) {
#pragma unroll
        for (int c = 0; c < kZL; ++c) {
            const int pl = c0 + c * ZG < a.nch ? c0 + c * ZG : 0;
            zq[c] = zsrc[size_t(pl) * E + q];
        }
    };
    auto zadd = [&](float& zsum, const float (&zq)[kZL], int c0) {
#pragma unroll
        for (int c = 0; c < kZL; ++c)
            if (c0 + c * ZG < a.nch) zsum += zq[c];
    };
    int zq0, zp0;
    const bool zon0 = a.r > 0 && zentry(0, zq0, zp0);
    float zfirst[kZL];
    zload(zfirst, a.r > 0 ? zp0 : 0, zon0 ? zq0 : 0);
    constexpr int kXPer = kSkinnyT * kMaxK / 8 / (kW * 64);  // 16-byte chunks per thread at most
    const int c8n = K / 8;
    u32x4 xv[kXPer];
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
        const int q = tid + k * kW * 64, t = q / c8n, c8 = (q % c8n) * 8;
        const bool on = q < kSkinnyT * c8n && t < T;
        xv[k] = *reinterpret_cast<const u32x4*>(a.x + (on ? size_t(t) * K + c8 : 0));
        if (!on) xv[k] = u32x4{0u, 0u, 0u, 0u};
    }
    float zv[2] = {0.f, 0.f};
    if (a.r > 0) {  // uniform
        float zsum = 0.f;
        zadd(zsum, zfirst, zp0);
        for (int c0 = zp0 + kZL * ZG; c0 < a.nch; c0 += kZL * ZG) {
            float zq[kZL];
            zload(zq, c0, zon0 ? zq0 : 0);
            zadd(zsum, zq, c0);
        }
        zv[0] = zon0 ? zsum : 0.f;
        if (ZG == 1 && E > kW * 64) {
            int q1, p1;
            const bool zon1 = zentry(1, q1, p1);
            float zsum1 = 0.f;
            for (int c0 = 0; c0 < a.nch; c0 += kZL) {
                float zq[kZL];
                zload(zq, c0, zon1 ? q1 : 0);
                zadd(zsum1, zq, c0);
            }
            zv[1] = zon1 ? zsum1 : 0.f;
        }
    }
    tab[trt][te * 32 + tc] = BITS == 2 ? (t0 | (t1 << 16)) : t0;
    if (ZG > 1) {
        if (tid < ZG * E) zpart[tid] = zv[0];  // class tid / E, entry tid % E
    } else {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (tid + k * kW * 64 < E) zpart[tid + k * kW * 64] = zv[k];
    }
    if (tid < nuc) *reinterpret_cast<u32x4*>(us + 8 * tid) = uv;
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
        const int q = tid + k * kW * 64, t = q / c8n, c8 = (q % c8n) * 8;
        if (q < kSkinnyT * c8n) *reinterpret_cast<u32x4*>(&xs[t][c8]) = xv[k];
    }
    __syncthreads();
    for (int q = tid; q < E; q += kW * 64) {
        float zsum = 0.f;
        for (int p = 0; p < ZG; ++p) zsum += zpart[p * E + q];
        zs[q] = zsum;
    }

    // ---- products
    const char* tbase = reinterpret_cast<const char*>(&tab[0][0]);
    const uint32_t lb = (uint32_t(l & 31) << 2) | uint32_t(rt * kTabDw * 4);
    const int n = l & 15;  // B column: token n
    const f32x4 acc = lut_products<BITS, FULL>(cw, nus, u0, g, tbase, lb, xs, n);
    red[w][l] = acc;
    __syncthreads();

    // ---- epilogue: thread (row tile, lane with token < 8, reg) sums the 8 slices, scales, adds
    // the rank-r term in FP32
    if (tid < 256) {
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < kKS; ++s) v += red[ert * kKS + s][el][eq];
        const int t = el & 15;
        if (t < T) {
            v *= h2f(escb);
            // rank-r term in FP32: the U row from LDS in chunks of 8
            float rs = 0.f;
            const float* zt = zs + t * a.r;
            const uint16_t* ur = us + (erow - row0) * a.r;
            for (int c = 0; 8 * c < a.r; ++c) {
                const u32x4 u8 = *reinterpret_cast<const u32x4*>(ur + 8 * c);
                const f32x4 z0 = *reinterpret_cast<const f32x4*>(zt + 8 * c);
                const f32x4 z1 = *reinterpret_cast<const f32x4*>(zt + 8 * c + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    rs += h2f(uint16_t(u8[e / 2] >> (16 * (e & 1)))) * (e < 4 ? z0[e] : z1[e - 4]);
            }
            v += rs;
            a.y[size_t(t) * N + erow] = uint16_t(f2h(v));
        }
    }
}

// ---- greedy argmax of a scalar-LUT output head (no rotation, no factors): y = sc . (W_lut x~)
// is never written; the largest logit of each token and its row are.  Persistent workgroups of
// the same shape as k_lut8 stage x~ once and walk the 32-row blocks b, b + G, ...; a block's code
// runs and table words are requested one block ahead (tables and partial sums double-buffered in
// LDS, one barrier per block: a block's epilogue runs beside the next block's products).  The
// epilogue keeps, per output thread, the best (value, row) seen (rows only grow, so a strictly
// larger value is needed to replace: the lowest row wins ties); at the end the workgroup's
// threads of a token are merged into part[b][t], and k_argmax_merge merges the workgroups.
template <int BITS, bool FULL>
__global__ void __launch_bounds__(kW * 64, 1) k_lut8_argmax(Lut8Args a, float* pval, int* pidx) {
    constexpr int CW = BITS == 2 ? 1 : 2;
    constexpr int kOffX = 2 * 2 * kTabDw * 4, kOffRed = kOffX + kSkinnyT * kXRow * 2;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kOffRed + 2 * kW * 64 * 16];
    auto& tab = *reinterpret_cast<uint32_t (*)[2][2][kTabDw]>(lds);  // [buffer][row tile][.]
    auto& xs = *reinterpret_cast<uint16_t (*)[kSkinnyT][kXRow]>(lds + kOffX);
    auto& red = *reinterpret_cast<f32x4 (*)[2][kW][64]>(lds + kOffRed);  // [buffer][wave][lane]
    float* mval = reinterpret_cast<float*>(lds + kOffRed);       // final merge (reuses red)
    int* midx = reinterpret_cast<int*>(lds + kOffRed + 256 * 4);

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, T = a.T, nb = a.N / 32, G = gridDim.x;
    const int rt = w / kKS, ks = w % kKS;
    const int nu = K / 64, u0 = ks * nu / kKS, nus = (ks + 1) * nu / kKS - u0;
    const int i = l & 15, g = l >> 4;
    constexpr int kRunW = kMaxU * CW, kRunV = (kRunW + 3) / 4;
    auto load_codes = [&](int blk, uint32_t (&cw)[kRunV * 4]) {
        const uint32_t* crun = a.codes + size_t(blk * 32 + rt * 16 + i) * (K * BITS / 32) +
                               u0 * (64 * BITS / 32) + g * nus * (16 * BITS / 32);
#pragma unroll
        for (int v = 0; v < kRunV; ++v) {
            const u32x4a q = *reinterpret_cast<const u32x4a*>(crun + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) cw[4 * v + e] = q[e];
        }
    };
    const int trt = tid >> 9, te = (tid >> 5) & 15, tc = tid & 31;
    auto load_tab = [&](int blk) -> uint32_t {
        const int grp = (blk * 32 + trt * 16) / 8 + ((tc & 15) >> 3);
        if constexpr (BITS == 2)
            return uint32_t(a.lut[grp * 4 + (te & 3)]) | (uint32_t(a.lut[grp * 4 + (te >> 2)]) << 16);
        else
            return a.lut[grp * 16 + te];
    };
    // epilogue thread: row tile, lane holding a token < 8, reg
    const int ert = tid >> 7, ej = tid & 127, ell = ej >> 2, eq = ej & 3;
    const int el = (ell >> 3) * 16 + (ell & 7), et = el & 15;
    const int erl = ert * 16 + 4 * (el >> 4) + eq;  // row within the block

    // every thread loads a scale (threads past the epilogue's 256 a harmless duplicate): a load
    // under a branch would have to complete inside it, and with in-order returns that wait
    // would also cover the code words requested before it
    const int erw = erl & 31;
    int blk = blockIdx.x;
    uint32_t tv = load_tab(blk);
    uint16_t esc = a.sc[blk * 32 + erw];
    uint32_t cw[kRunV * 4];
    load_codes(blk, cw);
    // x~ (rows past T zero), all loads before the stores
    constexpr int kXPer = kSkinnyT * kMaxK / 8 / (kW * 64);
    const int c8n = K / 8;
    {
        u32x4 xv[kXPer];
#pragma unroll
        for (int k = 0; k < kXPer; ++k) {
            const int q = tid + k * kW * 64, t = q / c8n, c8 = (q % c8n) * 8;
            xv[k] = q < kSkinnyT * c8n && t < T ? *reinterpret_cast<const u32x4*>(a.x + size_t(t) * K + c8)
                                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kXPer; ++k) {
            const int q = tid + k * kW * 64, t = q / c8n, c8 = (q % c8n) * 8;
            if (q < kSkinnyT * c8n) *reinterpret_cast<u32x4*>(&xs[t][c8]) = xv[k];
        }
    }
    const char* tb0 = reinterpret_cast<const char*>(&tab[0][0][0]);
    const int n = l & 15;
    float best = -__builtin_inff();
    int bidx = 0x7fffffff;
    // epilogue of block pblk from partials buffer pb: thread (row tile, lane holding a token < 8,
    // reg) sums the 8 slices, scales, and keeps a strictly larger value
    auto take = [&](int pb, int pblk, uint16_t pesc) {
        if (tid < 256) {
            float v = 0.f;
#pragma unroll
            for (int s = 0; s < kKS; ++s) v += red[pb][ert * kKS + s][el][eq];
            v *= h2f(pesc);
            if (v > best) {
                best = v;
                bidx = pblk * 32 + erl;
            }
        }
    };
    // The partials alternate between two buffers, so one barrier per block suffices: a block's
    // epilogue runs after the next block's barrier, beside that block's products.
    int pblk = -1, ppar = 0;
    uint16_t pesc = 0;
    for (int it = 0; blk < nb; ++it, blk += G) {
        const int par = it & 1;
        tab[par][trt][te * 32 + tc] = tv;
        // the next block's words, requested now (none after the workgroup's last block)
        const bool more = blk + G < nb;  // uniform
        uint32_t tvn = 0, cn[kRunV * 4];
        uint16_t escn = 0;
        if (more) {
            tvn = load_tab(blk + G);
            escn = a.sc[(blk + G) * 32 + erw];
            load_codes(blk + G, cn);
        }
        // this block's tables written; the last block's partials complete, and those of the
        // block before it (this buffer) consumed
        __syncthreads();
        if (pblk >= 0) take(ppar, pblk, pesc);
        const uint32_t lb = (uint32_t(l & 31) << 2) | uint32_t(((par * 2 + rt) * kTabDw) * 4);
        const f32x4 acc = lut_products<BITS, FULL>(cw, nus, u0, g, tb0, lb, xs, n);
        red[par][w][l] = acc;
        pblk = blk;
        ppar = par;
        pesc = esc;
        if (more) {
#pragma unroll
            for (int k = 0; k < kRunV * 4; ++k) cw[k] = cn[k];
            tv = tvn;
            esc = escn;
        }
    }
    __syncthreads();
    if (pblk >= 0) take(ppar, pblk, pesc);
    // merge the 32 threads of each token (2 row tiles x 4 lane groups x 4 regs): larger value,
    // then lower row
    __syncthreads();
    if (tid < 256) {
        mval[tid] = best;
        midx[tid] = bidx;
    }
    __syncthreads();
    if (tid < kSkinnyT) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
        for (int q = 0; q < 256; ++q) {
            const int qj = q & 127, qll = qj >> 2, qel = (qll >> 3) * 16 + (qll & 7);
            if ((qel & 15) != tid) continue;
            const float v = mval[q];
            const int ix = midx[q];
            if (v > bv || (v == bv && ix < bi)) {
                bv = v;
                bi = ix;
            }
        }
        pval[blockIdx.x * kSkinnyT + tid] = bv;
        pidx[blockIdx.x * kSkinnyT + tid] = bi;
    }
}

// merge of the workgroups' bests: 256 threads take candidates b = tid, tid + 256, ... (8 tokens
// each, two 16-byte loads), then a tree in LDS.  The order "larger value, then lower row" is a
// total order, so the winner does not depend on how the candidates are grouped.
__device__ __forceinline__ void argmax_take(float& bv, int& bi, float v, int ix) {
    if (v > bv || (v == bv && ix < bi)) {
        bv = v;
        bi = ix;
    }
}
__global__ void __launch_bounds__(256) k_argmax_merge(int G, int T, const float* pval, const int* pidx,
                                                      int* out_idx, float* out_val) {
    __shared__ float sv[kSkinnyT][256];
    __shared__ int si[kSkinnyT][256];
    const int tid = threadIdx.x;
    float bv[kSkinnyT];
    int bi[kSkinnyT];
#pragma unroll
    for (int t = 0; t < kSkinnyT; ++t) {
        bv[t] = -__builtin_inff();
        bi[t] = 0x7fffffff;
    }
    for (int b = tid; b < G; b += 256) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(pval + b * kSkinnyT);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(pval + b * kSkinnyT + 4);
        const u32x4 i0 = *reinterpret_cast<const u32x4*>(pidx + b * kSkinnyT);
        const u32x4 i1 = *reinterpret_cast<const u32x4*>(pidx + b * kSkinnyT + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            argmax_take(bv[t], bi[t], v0[t], int(i0[t]));
            argmax_take(bv[t + 4], bi[t + 4], v1[t], int(i1[t]));
        }
    }
#pragma unroll
    for (int t = 0; t < kSkinnyT; ++t) {
        sv[t][tid] = bv[t];
        si[t][tid] = bi[t];
    }
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) {
#pragma unroll
            for (int t = 0; t < kSkinnyT; ++t) {
                float v = sv[t][tid];
                int ix = si[t][tid];
                argmax_take(v, ix, sv[t][tid + h], si[t][tid + h]);
                sv[t][tid] = v;
                si[t][tid] = ix;
            }
        }
        __syncthreads();
    }
    if (tid < T) {
        out_idx[tid] = si[tid][0];
        if (out_val) out_val[tid] = sv[tid][0];
    }
}

int lut8_argmax_grid(int N, int cus) {
    const int nb = N / 32;
    return nb < cus ? nb : cus;
}

hipError_t launch_lut8_argmax(const Lut8Args& a, int cus, float* pval, int* pidx, int* out_idx,
                              float* out_val, hipStream_t st) {
    if (!a.codes || !a.lut || !a.sc || !a.x || !pval || !pidx || !out_idx ||
        (a.bits != 2 && a.bits != 4) || a.N < 32 || a.N % 32 || a.K < 64 || a.K % 64 ||
        a.K > kMaxK || a.T < 1 || a.T > kSkinnyT || a.r != 0 || cus < 1)
        return hipErrorInvalidValue;
    const int G = lut8_argmax_grid(a.N, cus);
    const bool full = a.K == kMaxK;  // every K slice holds kMaxU units
#define VQ_ARGMAX(B, F) hipLaunchKernelGGL((k_lut8_argmax<B, F>), dim3(G), dim3(kW * 64), 0, st, a, pval, pidx)
    if (a.bits == 2 && full)
        VQ_ARGMAX(2, true);
    else if (a.bits == 2)
        VQ_ARGMAX(2, false);
    else if (full)
        VQ_ARGMAX(4, true);
    else
        VQ_ARGMAX(4, false);
#undef VQ_ARGMAX
    hipLaunchKernelGGL(k_argmax_merge, dim3(1), dim3(256), 0, st, G, a.T, pval, pidx, out_idx, out_val);
    return hipGetLastError();
}

// ---- pre-pass: workgroup (chunk c of C = 64 V columns, group of 16 rows of V, part p of the
// chunk's CS = min(C, 256) columns); wave t < 8 holds token row t of the whole chunk, V
// consecutive columns per lane (16-byte loads of x, s, sign).  The Walsh-Hadamard butterflies
// (blocks of hb, distances 1 .. hb/2 in that order, each pair (lo, hi) -> (lo + hi, lo - hi)) run
// in registers below V and across lanes above (lane_xor: DPP moves for distances of 1, 2 and 8
// lanes, swizzles for 4 and 16, a permute for 32);
// x~ = . / sqrt(hb) is rounded to binary16, written out by the chunk's first workgroup and kept
// in LDS for the part's columns, where the group's 16 rows of V (one 16-byte load per thread,
// issued first) meet it on the matrix cores: wave w takes the 32-column steps w, w + 8, ... (A =
// 16 rows of V, B = x~, column n = token n, zero for n >= 8).  Partial sums of z go to plane
// c * (C / CS) + p.
template <int V>
__global__ void __launch_bounds__(512) k_lut8_pre(int T, int K, int hb, const uint16_t* x,
                                                  const uint16_t* s, const int8_t* sign,
                                                  const uint16_t* Vm, int r, uint16_t* xt,
                                                  float* zp, float norm) {
    constexpr int C = 64 * V, CS = C < 256 ? C : 256, XR = CS + 8;
    __shared__ __attribute__((aligned(16))) uint16_t vs[16 * CS];
    __shared__ __attribute__((aligned(16))) uint16_t xh[kSkinnyT * XR];
    __shared__ f32x4 zred[8][64];
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int c = blockIdx.x, rg = blockIdx.y, part = blockIdx.z;
    const int c0 = c * C, col = c0 + V * l;
    // the group's V rows over the part's columns: 16 x CS in 16-byte chunks, issued first
    u32x4 vv = u32x4{0u, 0u, 0u, 0u};
    if (r > 0 && tid < 2 * CS) {
        const int jr = tid / (CS / 8), cc = (tid % (CS / 8)) * 8;
        vv = *reinterpret_cast<const u32x4*>(Vm + size_t(rg * 16 + jr) * K + c0 + part * CS + cc);
    }
    // row w of x . s . sign
    float v[V];
    {
        const int t = w;
#pragma unroll
        for (int q = 0; q < (V + 7) / 8; ++q) {
            constexpr int kE = V < 8 ? V : 8;
            uint32_t xw[4] = {0u, 0u, 0u, 0u}, sw[4] = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
            uint64_t gw = 0;
            if (t < T) {
                if constexpr (kE == 8) {
                    const u32x4 a4 = *reinterpret_cast<const u32x4*>(x + size_t(t) * K + col + 8 * q);
                    for (int e = 0; e < 4; ++e) xw[e] = a4[e];
                    if (s) {
                        const u32x4 s4 = *reinterpret_cast<const u32x4*>(s + col + 8 * q);
                        for (int e = 0; e < 4; ++e) sw[e] = s4[e];
                    }
                    if (sign) gw = *reinterpret_cast<const uint64_t*>(sign + col + 8 * q);
                } else {
                    for (int e = 0; e < kE; ++e) {
                        xw[e / 2] |= uint32_t(x[size_t(t) * K + col + e]) << (16 * (e & 1));
                        if (s) sw[e / 2] = (sw[e / 2] & ~(0xFFFFu << (16 * (e & 1)))) |
                                           (uint32_t(s[col + e]) << (16 * (e & 1)));
                        if (sign) gw |= uint64_t(uint8_t(sign[col + e])) << (8 * e);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                float u = h2f(uint16_t(xw[e / 2] >> (16 * (e & 1)))) * h2f(uint16_t(sw[e / 2] >> (16 * (e & 1))));
                if (int8_t(gw >> (8 * e)) < 0) u = -u;
                v[8 * q + e] = t < T ? u : 0.f;
            }
        }
    }
#pragma unroll
    for (int h = 1; h < V; h <<= 1)
        if (h < hb) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (!(e & h)) {
                    const float x0 = v[e], x1 = v[e | h];
                    v[e] = x0 + x1;
                    v[e | h] = x0 - x1;
                }
        }
    // across lanes: distance V d pairs lane l with l ^ d; the upper lane takes (lo - hi) as
    // partner - own, the lower one own + partner (a multiply by -1 or 1 is exact, so the fused
    // form rounds as the plain sum does)
#define VQ_PRE_STAGE(DD)                                                \
    if (V * DD < hb) {                                                  \
        const float sg = (l & DD) ? -1.f : 1.f;                         \
        _Pragma("unroll") for (int e = 0; e < V; ++e)                   \
            v[e] = __builtin_fmaf(v[e], sg, lane_xor<DD>(v[e]));        \
    }
    VQ_PRE_STAGE(1) VQ_PRE_STAGE(2) VQ_PRE_STAGE(4) VQ_PRE_STAGE(8) VQ_PRE_STAGE(16) VQ_PRE_STAGE(32)
#undef VQ_PRE_STAGE
    uint32_t hp[(V + 1) / 2];
#pragma unroll
    for (int e = 0; e < V; e += 2)
        hp[e / 2] = f2h(v[e] * norm) | (e + 1 < V ? f2h(v[e + 1] * norm) << 16 : 0u);
    if (rg == 0 && part == 0 && w < T) {
        uint16_t* dst = xt + size_t(w) * K + col;
        if constexpr (V >= 8) {
#pragma unroll
            for (int q = 0; q < V / 8; ++q)
                *reinterpret_cast<u32x4*>(dst + 8 * q) = u32x4{hp[4 * q], hp[4 * q + 1], hp[4 * q + 2], hp[4 * q + 3]};
        } else if constexpr (V >= 2) {
#pragma unroll
            for (int q = 0; q < V / 2; ++q) *reinterpret_cast<uint32_t*>(dst + 2 * q) = hp[q];
        } else {
            *dst = uint16_t(hp[0]);
        }
    }
    if (r == 0) return;
    // z is formed from the rounded x~, as the product reads it: the part's columns into LDS
    const int lc = V * l - part * CS;
    if (lc >= 0 && lc < CS) {
#pragma unroll
        for (int e = 0; e < V; e += 2) {
            if (V >= 2)
                *reinterpret_cast<uint32_t*>(&xh[w * XR + lc + e]) = hp[e / 2];
            else
                xh[w * XR + lc] = uint16_t(hp[0]);
        }
    }
    if (tid < 2 * CS) *reinterpret_cast<u32x4*>(&vs[(tid / (CS / 8)) * CS + (tid % (CS / 8)) * 8]) = vv;
    __syncthreads();
    const int i = l & 15, g = l >> 4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 32 * w; kk < CS; kk += 256) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(&vs[i * CS + kk + 8 * g]);
        const u32x4 B = i < kSkinnyT ? *reinterpret_cast<const u32x4*>(&xh[(i < kSkinnyT ? i : 0) * XR + kk + 8 * g])
                                     : u32x4{0u, 0u, 0u, 0u};
        acc = mfma16x16x32(A, B, acc);
    }
    zred[w][l] = acc;
    __syncthreads();
    if (tid < 256) {
        // lane ll holds rows 4 (ll / 16) + q of the block, token ll % 16
        const int ll = tid >> 2, q = tid & 3, t = ll & 15, jl = 4 * (ll >> 4) + q;
        if (t < kSkinnyT) {
            float sum = 0.f;
#pragma unroll
            for (int ww = 0; ww < 8; ++ww) sum += zred[ww][ll][q];
            const int pl = c * (C / CS) + part;
            zp[(size_t(pl) * kSkinnyT + t) * r + rg * 16 + jl] = sum;
        }
    }
}

int lut8_chunk(int K, int hb) {
    // the widest power-of-two chunk of 64 .. 1024 columns that is a whole number of Hadamard
    // blocks and divides K (0: none)
    const int b = hb > 1 ? hb : 1;
    int best = 0;
    for (int c = 64; c <= 1024; c *= 2)
        if (K % c == 0 && c % b == 0) best = c;
    return best;
}

int lut8_planes(int K, int hb) {
    const int C = lut8_chunk(K, hb);
    return C < 64 ? 0 : K / (C < 256 ? C : 256);
}

hipError_t launch_lut8_pre(int T, int K, int hb, const uint16_t* x, const uint16_t* s,
                           const int8_t* sign, const uint16_t* V, int r, uint16_t* xt, float* zp,
                           hipStream_t st) {
    const int C = lut8_chunk(K, hb);
    if (!x || !xt || C < 64 || T < 1 || T > kSkinnyT || r < 0 || r % 16 || (r > 0 && (!V || !zp)) ||
        hb < 1 || hb > 1024 || (hb & (hb - 1)))
        return hipErrorInvalidValue;
    const float norm = float(1.0 / __builtin_sqrt(double(hb)));
    // z's parts: chunks of more than 256 columns are cut in 256-column parts (one workgroup each)
    const dim3 grid(K / C, r > 0 ? r / 16 : 1, r > 0 && C > 256 ? C / 256 : 1);
#define VQ_PRE(VV)                                                                                \
    if (C == 64 * VV) {                                                                           \
        hipLaunchKernelGGL(k_lut8_pre<VV>, grid, dim3(512), 0, st, T, K, hb, x, s, sign, V, r, xt, \
                           zp, norm);                                                             \
        return hipGetLastError();                                                                 \
    }
    VQ_PRE(1) VQ_PRE(2) VQ_PRE(4) VQ_PRE(8) VQ_PRE(16)
#undef VQ_PRE
    return hipErrorInvalidValue;
}

hipError_t launch_lut8(const Lut8Args& a, hipStream_t st) {
    if (!a.codes || !a.lut || !a.sc || !a.x || !a.y || (a.bits != 2 && a.bits != 4) || a.N < 32 ||
        a.N % 32 || a.K < 64 || a.K % 64 || a.K > kMaxK || a.T < 1 || a.T > kSkinnyT || a.r < 0 ||
        a.r > kMaxR || a.r % 8 || (a.r > 0 && (!a.U || !a.zp || a.nch < 1)))
        return hipErrorInvalidValue;
    const bool full = a.K == kMaxK;  // every K slice holds kMaxU units
#define VQ_LUT8(B, F) hipLaunchKernelGGL((k_lut8<B, F>), dim3(a.N / 32), dim3(kW * 64), 0, st, a)
    if (a.bits == 2 && full)
        VQ_LUT8(2, true);
    else if (a.bits == 2)
        VQ_LUT8(2, false);
    else if (full)
        VQ_LUT8(4, true);
    else
        VQ_LUT8(4, false);
#undef VQ_LUT8
    return hipGetLastError();
}

}  // namespace vqmlp
