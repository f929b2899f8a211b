// vq3mm.hip -- matrix-core product with the VQ3 weights decoded in registers, for T > 64 rows
// (gfx950).
//
//   D[t][n] = sum_k X[t][k] W[n][k],   X binary16 [T][K] (rotated activations), W packed VQ3.
//
// Model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP, token-mixer
// rotations, distilled weights": a six-bit code selects the pair (W[2p][j], W[2p+1][j]) from 64
// two-component binary16 centroids shared by 8 rows; row scales are applied in the epilogue.
//
// Work split.  A workgroup of NW waves owns BM tokens x NW*RW rows (of each of NMAT matrices that
// share X).  Each wave owns RW rows and all BM tokens, so no weight is used by two waves and the
// weights never pass through LDS: a wave decodes its own codes straight into the B operand of
// v_mfma_f32_16x16x32_f16.  Only the activation tile is staged through LDS, where all waves read it.
//
// Decoding one 16-row x 32-column B operand.  A group's 64 centroids sit in one register (lane e
// holds centroid e), and a cross-lane read (ds_bpermute) returns one centroid per lane.  The
// operand spans two groups (rows 0-7 and 8-15) and every centroid holds halves for two rows, so
// the operand's 256 centroids come in four reads -- two from each group's register, every lane
// reading for itself or for lane n ^ 8 -- followed by two exchanges: lanes n and n ^ 8 trade the
// other group's centroids (DPP row rotate by 8 with a bank mask), then lanes n and n ^ 1 trade
// the other row's halves (DPP quad permute).
//
// Column order.  Within a 64-column K tile, operand slot (ks, kg, i) -- K step ks (of 2), lane
// group kg = lane / 16, element i (of 8) -- holds column 16 (i / 2) + 4 kg + 2 ks + (i % 2).  With
// this order each lane's codes for a K tile are one 24-bit slot of two 96-bit lane records of the
// packed tile (slot s of the records of its own pair and of the pair four up).  The activations
// are staged into LDS in the same order, so an A operand is still one 16-byte LDS read.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace vqmlp {

namespace {

constexpr int kXK = 64;   // K tile
constexpr int kXLd = 72;  // LDS row stride of the activation tile (halves)

constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3: 32-bit raw data
constexpr int kDppRor8 = 0x128;  // row_ror:8 -- lane n of each 16-lane row reads lane n ^ 8
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2] -- lane n reads lane n ^ 1

__device__ __forceinline__ uint32_t bperm(uint32_t byte_addr, uint32_t v) {
    // the source lane is bits 7:2 of the address; higher bits are ignored
    return uint32_t(__builtin_amdgcn_ds_bpermute(int(byte_addr), int(v)));
}
// lanes of the banks in BANKS (4 lanes per bank, 4 banks per 16-lane row) take src from lane
// n ^ 8; the others keep old
template <int BANKS>
__device__ __forceinline__ uint32_t ror8_into(uint32_t old, uint32_t src) {
    return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(src), kDppRor8, 0xF, BANKS, false));
}
__device__ __forceinline__ uint32_t from_xor1(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), kDppXor1, 0xF, 0xF, false));
}

template <int NW, int BM, int RW, int NMAT, int EPI>
__global__ void __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_vq3mm(GemmArgs a) {
    constexpr int NT = NW * 64;
    constexpr int RF = RW / 16;   // 16-row operands per wave per matrix
    constexpr int TF = BM / 16;   // 16-token operands
    constexpr int CT = RW / 32;   // packed 32-row code tiles per wave per matrix
    constexpr int BNW = NW * RW;  // rows per workgroup
    constexpr int XCH = BM * 8 / NT;  // 16-byte activation chunks per thread per K tile
    static_assert(RW % 32 == 0 && XCH >= 1 && (BM * 8) % NT == 0, "shape");
    constexpr int kXBytes = 2 * BM * kXLd * 2;
    constexpr int kEpBytes = EPI == kEgGateUpRot ? BM * (BNW + 1) * 4 : 0;
    constexpr int kLds = kXBytes > kEpBytes ? kXBytes : kEpBytes;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
    auto& Xs = *reinterpret_cast<uint16_t (*)[2][BM][kXLd]>(lds);

    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int n = l & 15, kg = l >> 4, c0 = n & 1, s = c0 + 2 * (n >> 3), pb = (n >> 1) & 3;
    const int N = a.N, K = a.K, T = a.T, KT = K / kXK;
    const int row0 = blockIdx.x * BNW, tok0 = blockIdx.y * BM;
    const int wrow = row0 + w * RW;  // first row of this wave
    const int ldo = a.ldo > 0 ? a.ldo : N;
    const int mt_last = N / 32 - 1;

    // ---- centroids: one register per 8-row group, lane e holds centroid e
    uint32_t cbr[NMAT][RW / 8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int g = 0; g < RW / 8; ++g) {
            const int grp = min(wrow / 8 + g, N / 8 - 1);
            cbr[m][g] = a.cb[m][size_t(grp) * 64 + l];
        }

    // ---- this lane's code words: for operand j (rows wrow + 16 j ..) the records of pair
    // 8 (j % 2) + pb (rows of the first group) and of that pair + 4 (second group), lane-record
    // column group kg; the two words holding 24-bit slot s (words 0, 1 for s < 2, else 1, 2).
    uint32_t voff[RF][2];
#pragma unroll
    for (int j = 0; j < RF; ++j) {
        const int mt = min(wrow / 32 + j / 2, mt_last);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int pp = 8 * (j & 1) + 4 * h + pb;
            voff[j][h] = uint32_t(mt) * uint32_t(KT) * kTileBytes + 12u * uint32_t((kg << 4) | pp) +
                         4u * uint32_t(s >> 1);
        }
    }
    const uint32_t sh24 = uint32_t(24 * s) & 31u;
    const bool s3 = s == 3;
    // v_perm selectors: this lane's row half (component c0) and the partner's
    const uint32_t sel_own = c0 ? 0x07060302u : 0x05040100u;
    const uint32_t sel_oth = c0 ? 0x05040100u : 0x07060302u;

    // Loads go through buffer resources: the lane's offset is fixed for the whole K loop and the
    // K tile's offset rides in the scalar offset, so no address arithmetic is spent per load.
    __amdgpu_buffer_rsrc_t rs_code[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        rs_code[m] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>((NMAT > 1 && m) ? a.codes[1] : a.codes[0]), 0,
            int(uint32_t(N / 32) * uint32_t(KT) * kTileBytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x), 0, int(uint32_t(T) * uint32_t(K) * 2u), kRsrcWord3);
    uint32_t xoff[XCH];  // byte offset of this thread's activation chunk in K tile 0
#pragma unroll
    for (int x = 0; x < XCH; ++x) {
        const int c = tid + x * NT;
        const int tok = min(tok0 + (c >> 3), T - 1);  // rows past T are zeroed at staging
        xoff[x] = (uint32_t(tok) * uint32_t(K) + 8u * uint32_t(c & 7)) * 2u;
    }

    u32x4 xr[2][XCH];            // activation chunks of two K tiles in flight
    u32x2 cw[2][NMAT][RF][2];    // code words of two K tiles in flight
    u32x4 Bf[2][2][NMAT][RF];    // decoded B operands of two K tiles: [tile parity][ks][m][j]

    auto load_x = [&](int kt, int set) {
#pragma unroll
        for (int x = 0; x < XCH; ++x)
            xr[set][x] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, int(xoff[x]), kt * kXK * 2, 0));
    };
    auto load_codes = [&](int kt, int set) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    cw[set][m][j][h] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs_code[m], int(voff[j][h]),
                                                                    kt * kTileBytes, 0));
    };

    // 16-byte chunk u of a token's 64 columns (columns 8u .. 8u+7) goes to operand positions
    // base, base+32, base+8, base+40 (one word each), base = 16 (u % 2) + 2 (u / 2)
    auto stage = [&](int buf, int set) {
#pragma unroll
        for (int x = 0; x < XCH; ++x) {
            const int c = tid + x * NT;
            const int tt = c >> 3, u = c & 7;
            // all-ones for tokens below T: a mask keeps the stores unconditional
            const uint32_t keep = 0u - uint32_t(tok0 + tt < T);
            uint32_t* row = reinterpret_cast<uint32_t*>(&Xs[buf][tt][0]);
            const int b2 = 8 * (u & 1) + (u >> 1);
            row[b2] = xr[set][x][0] & keep;
            row[b2 + 16] = xr[set][x][1] & keep;
            row[b2 + 4] = xr[set][x][2] & keep;
            row[b2 + 20] = xr[set][x][3] & keep;
        }
    };

    // the lane's 24-bit code slot of every record (codes q = 0..3 at bits 6q)
    uint32_t c24[NMAT][RF][2];
    auto extract = [&](int set) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x2 v = cw[set][m][j][h];
                    c24[m][j][h] = __builtin_amdgcn_alignbit(v[1], s3 ? v[1] : v[0], sh24);
                }
    };
    // Decoding unit u = (ks, m, j) of the B operands (U of them per K tile), in two phases: the
    // four cross-lane centroid reads, then the exchanges that place the halves.
    constexpr int U = 2 * NMAT * RF;
    uint32_t ev[2][4];  // centroid reads of two units in flight
    auto dec_read = [&](int u) {
        const int ks = u / (NMAT * RF), m = (u / RF) % NMAT, j = u % RF;
        // codes q = 2 ks, 2 ks + 1 moved to address bits 7:2
        const uint32_t ca = c24[m][j][0], cb = c24[m][j][1];
        const uint32_t a0 = ks ? ca >> 10 : ca << 2, a1 = ks ? ca >> 16 : ca >> 4;
        const uint32_t b0 = ks ? cb >> 10 : cb << 2, b1 = ks ? cb >> 16 : cb >> 4;
        ev[u & 1][0] = bperm(a0, cbr[m][2 * j]);
        ev[u & 1][1] = bperm(a1, cbr[m][2 * j]);
        ev[u & 1][2] = bperm(b0, cbr[m][2 * j + 1]);
        ev[u & 1][3] = bperm(b1, cbr[m][2 * j + 1]);
    };
    auto dec_place = [&](int u, int par) {
        const int ks = u / (NMAT * RF), m = (u / RF) % NMAT, j = u % RF;
        const uint32_t e0 = ev[u & 1][0], e1 = ev[u & 1][1], e2 = ev[u & 1][2], e3 = ev[u & 1][3];
        // lanes 0-7 keep their own group's centroids, lanes 8-15 take them from n - 8 (low
        // column block); the high block the other way round
        const uint32_t lo0 = ror8_into<0xC>(e0, e2), hi0 = ror8_into<0x3>(e2, e0);
        const uint32_t lo1 = ror8_into<0xC>(e1, e3), hi1 = ror8_into<0x3>(e3, e1);
        const uint32_t ylo = __builtin_amdgcn_perm(lo1, lo0, sel_own);
        const uint32_t zlo = from_xor1(__builtin_amdgcn_perm(lo1, lo0, sel_oth));
        const uint32_t yhi = __builtin_amdgcn_perm(hi1, hi0, sel_own);
        const uint32_t zhi = from_xor1(__builtin_amdgcn_perm(hi1, hi0, sel_oth));
        Bf[par][ks][m][j] = c0 ? u32x4{zlo, ylo, zhi, yhi} : u32x4{ylo, zlo, yhi, zhi};
    };
    auto build = [&](int par) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            dec_read(u);
            dec_place(u, par);
        }
    };

    f32x4 acc[NMAT][RF][TF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < RF; ++j)
#pragma unroll
            for (int i = 0; i < TF; ++i) acc[m][j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto readA = [&](int buf, int c) {  // A operand of product unit c = (ks, i)
        const int ks = c / TF, i = c % TF;
        return *reinterpret_cast<const u32x4*>(&Xs[buf][16 * i + n][32 * ks + 8 * kg]);
    };
    auto mma_unit = [&](int c, int par, const u32x4& A) {
        const int ks = c / TF, i = c % TF;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j) acc[m][j][i] = mfma16x16x32(A, Bf[par][ks][m][j], acc[m][j][i]);
    };
    auto mma = [&](int buf, int par) {
#pragma unroll
        for (int c = 0; c < 2 * TF; ++c) mma_unit(c, par, readA(buf, c));
    };

    // this workgroup's K tiles: split blockIdx.z of a.ksplit equal ranges
    const int nsplit = a.ksplit > 1 ? a.ksplit : 1;
    const int kb = int(blockIdx.z) * KT / nsplit, nk = (int(blockIdx.z) + 1) * KT / nsplit - kb;
    auto tile = [&](int t) { return kb + min(t, nk - 1); };  // loads past the end repeat the last

    // Software pipeline over K tiles t: while the matrix cores multiply tile t (activations from
    // LDS buffer t % 2, weights decoded one step earlier), the wave decodes tile t + 1's codes
    // (requested two steps earlier) and stages tile t + 1's activations; the code words of tile
    // t + 3 and the activations of tile t + 3 are requested as soon as their registers are free.
    // Every load is unconditional, so each wait counts the same loads on every path.
    load_codes(tile(0), 0);
    load_x(tile(0), 0);
    load_codes(tile(1), 1);
    load_x(tile(1), 1);
    stage(0, 0);
    extract(0);
    load_codes(tile(2), 0);
    load_x(tile(2), 0);
    build(0);
    __syncthreads();
    // One K step, hand-interleaved: product unit c (one A operand, NMAT x RF matrix-core steps)
    // alternates with the decoding of the next tile's B operands -- the placing of unit u and
    // the centroid reads of unit u + 1 -- so that the matrix cores, the VALU and the LDS work
    // side by side.  A operands are read two units ahead.  Scheduling barriers keep the order.
    constexpr int MU = 2 * TF;  // product units per K tile
    static_assert(MU % U == 0, "whole product units per decoding unit");
    auto step = [&](auto P, int t) {
        constexpr int p = decltype(P)::value;  // parity of tile t
        extract(1 - p);                       // codes of tile t + 1
        load_codes(tile(t + 3), 1 - p);
        u32x4 Ar[3];
        Ar[0] = readA(p, 0);
        Ar[1] = readA(p, 1);
        dec_read(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < MU; ++c) {
            if (c + 2 < MU) Ar[(c + 2) % 3] = readA(p, c + 2);
            mma_unit(c, p, Ar[c % 3]);
            if (c % (MU / U) == 0) {
                const int u = c / (MU / U);
                dec_place(u, 1 - p);
                if (u + 1 < U) dec_read(u + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        stage(1 - p, 1 - p);                  // activations of tile t + 1
        load_x(tile(t + 3), 1 - p);
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < nk; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < nk) mma(0, 0);

    // ---- epilogues.  Lane l, register q of acc[m][j][i] holds D[token][row] with
    // token = tok0 + 16 i + 4 kg + q and row = wrow + 16 j + n.
    if constexpr (EPI == kEgGateUpRot) {
        // a = silu(g) u sign over BM tokens x BNW rows in LDS (fp32), then the Hadamard transform
        // of every 128-row block, then binary16 out
        static_assert(NMAT == 2 && BNW % 128 == 0, "gate+up, whole rotation blocks");
        float* Ab = reinterpret_cast<float*>(lds);  // [BM][BNW + 1]
#pragma unroll
        for (int j = 0; j < RF; ++j) {
            const int rl = w * RW + 16 * j + n;
            const int row = min(row0 + rl, N - 1);
            const float sg = h2f(a.sc[0][row]), su = h2f(a.sc[1][row]);
            const bool neg = a.sign && a.sign[row] < 0;
#pragma unroll
            for (int i = 0; i < TF; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int tl = 16 * i + 4 * kg + q;
                    const float g = acc[0][j][i][q] * sg, u = acc[1][j][i][q] * su;
                    const float v = g / (1.f + expf(-g)) * u;
                    Ab[tl * (BNW + 1) + rl] = neg ? -v : v;
                }
        }
        __syncthreads();
        for (int h = 1; h < 128; h <<= 1) {
            for (int e = tid; e < BM * (BNW / 2); e += NT) {
                const int tl = e / (BNW / 2), jj = e % (BNW / 2);
                const int lo = (jj / h) * 2 * h + (jj % h), hi = lo + h;
                const float x0 = Ab[tl * (BNW + 1) + lo], x1 = Ab[tl * (BNW + 1) + hi];
                Ab[tl * (BNW + 1) + lo] = x0 + x1;
                Ab[tl * (BNW + 1) + hi] = x0 - x1;
            }
            __syncthreads();
        }
        for (int e = tid; e < BM * BNW / 2; e += NT) {
            const int tl = e / (BNW / 2), cc = (e % (BNW / 2)) * 2;
            const int tok = tok0 + tl;
            if (tok < T && row0 + cc < N) {
                const uint32_t hv = f2h(Ab[tl * (BNW + 1) + cc] * a.norm) |
                                    (f2h(Ab[tl * (BNW + 1) + cc + 1] * a.norm) << 16);
                *reinterpret_cast<uint32_t*>(a.out16 + size_t(tok) * ldo + row0 + cc) = hv;
            }
        }
        return;
    }

#pragma unroll
    for (int j = 0; j < RF; ++j) {
        const int row = wrow + 16 * j + n;
        if (wrow + 16 * j >= N) continue;  // whole 16-row operands (N is a multiple of 32)
        float s0 = 1.f, s1 = 1.f;
        bool neg = false;
        if constexpr (EPI == kEgGateUp32) {
            s0 = h2f(a.sc[0][row]);
            s1 = h2f(a.sc[1][row]);
            neg = a.sign && a.sign[row] < 0;
        } else if constexpr (EPI == kEgScale16) {
            s0 = h2f(a.sc[0][row]);
        }
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int tok = tok0 + 16 * i + 4 * kg + q;
                if (tok >= T) continue;
                const float v0 = acc[0][j][i][q];
                if constexpr (EPI == kEgGateUp32) {
                    const float g = v0 * s0, u = acc[NMAT - 1][j][i][q] * s1;
                    const float act = g / (1.f + expf(-g)) * u;
                    a.out32[size_t(tok) * ldo + row] = neg ? -act : act;
                } else if constexpr (EPI == kEgScale16) {
                    a.out16[size_t(tok) * ldo + row] = (uint16_t)f2h(v0 * s0);
                } else if constexpr (EPI == kEgPart2) {
                    // split z of a K-split gate/up product: unscaled g and u planes
                    float* o = a.out32 + (size_t(blockIdx.z) * T + tok) * 2 * N + row;
                    o[0] = v0;
                    o[N] = acc[NMAT - 1][j][i][q];
                } else {  // split z of a K-split product writes its own [T][N] plane
                    a.out32[(size_t(blockIdx.z) * T + tok) * N + row] = v0;
                }
            }
    }
}

template <int NW, int BM, int RW, int NMAT, int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
    constexpr int BNW = NW * RW;
    const dim3 grid((a.N + BNW - 1) / BNW, (a.T + BM - 1) / BM, a.ksplit > 1 ? a.ksplit : 1);
    hipLaunchKernelGGL((k_vq3mm<NW, BM, RW, NMAT, EPI>), grid, dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

// Tile shapes: waves, tokens and rows per wave of the gate/up product (two matrices) and of the
// down product (one matrix).  One wave per SIMD: the accumulators live in the AGPRs.
#ifndef VQ3MM_GU_NW
#define VQ3MM_GU_NW 4
#endif
#ifndef VQ3MM_GU_RW
#define VQ3MM_GU_RW 32
#endif
#ifndef VQ3MM_DN_NW
#define VQ3MM_DN_NW 4
#endif
#ifndef VQ3MM_DN_RW
#define VQ3MM_DN_RW 64
#endif
constexpr int kGuNW = VQ3MM_GU_NW, kGuBM = 128, kGuRW = VQ3MM_GU_RW;
constexpr int kDnNW = VQ3MM_DN_NW, kDnBM = 128, kDnRW = VQ3MM_DN_RW;

}  // namespace

Vq3Tile vq3mm_tile(int nmat) {
    return nmat == 2 ? Vq3Tile{kGuBM, kGuNW * kGuRW} : Vq3Tile{kDnBM, kDnNW * kDnRW};
}

hipError_t launch_vq3mm(const GemmArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.K % kXK || a.N <= 0 || a.N % 32) return hipErrorInvalidValue;
    if (a.ksplit > 1 && (a.K / kXK) < a.ksplit) return hipErrorInvalidValue;
    switch (a.kind) {
        case kGemmVQ3GateUp:
            return launch_t<kGuNW, kGuBM, kGuRW, 2, kEgGateUp32>(a, st);
        case kGemmVQ3GateUpRot:  // whole 128-row rotation blocks
            if (a.N % 128) return hipErrorInvalidValue;
            return launch_t<kGuNW, kGuBM, kGuRW, 2, kEgGateUpRot>(a, st);
        case kGemmVQ3GateUpSplit:
            return launch_t<kGuNW, kGuBM, kGuRW, 2, kEgPart2>(a, st);
        case kGemmVQ3Down:
            return launch_t<kDnNW, kDnBM, kDnRW, 1, kEgScale16>(a, st);
        case kGemmVQ3DownSplit:
            return launch_t<kDnNW, kDnBM, kDnRW, 1, kEgPlain32>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace vqmlp
