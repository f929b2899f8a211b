// tiled.hip -- matrix-core GEMM with on-the-fly weight decoding, for T > 8 rows (gfx950).
//
//   D[t][n] = sum_k X[t][k] W[n][k],   X binary16 [T][K] (rotated activations), W decoded per tile.
//
// Decoders (one 64-column K tile of BN rows at a time, into LDS as binary16):
//   VQ3   model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP,
//         token-mixer rotations, distilled weights": six-bit codes select (W[2p][j], W[2p+1][j])
//         from 64 two-component centroids per 8 rows (the packed tile layout of the library);
//   LUT2 / LUT4   same card, format table row "Token mixers": two- and four-bit lookup tables,
//         one table of 2^bits binary16 scalars per 8 rows;
//   VQ2   same card, format table, "Previous packages" column: the 2x16 vector LUT, four-bit
//         codes selecting (W[2p][j], W[2p+1][j]) from 16 two-component centroids per 8 rows
//         (codes row-major by row pair, 8 to a 32-bit word);
//   DENSE binary16 rows (the rank-r factor V).
// Row scales are applied to the accumulators in the epilogue (exact in real arithmetic).
//
// Work: a workgroup of 8 waves owns BM tokens x BN rows (of each of NMAT matrices sharing X).
// Waves form a 2 x 4 grid; each wave holds (BM/2) x (BN/4) outputs per matrix as 16x16 fp32
// tiles of v_mfma_f32_16x16x32_f16.  The K loop is double-buffered: while the matrix cores work
// on tile k from LDS, the raw bytes of tile k+1 are already in registers and are decoded into
// the other LDS buffer afterwards.
#include "device.h"
#include "internal.h"

#include <cmath>

namespace vqmlp {

constexpr int kGK = 64;        // K tile
constexpr int kGPad = 8;       // LDS row padding (halves)
constexpr int kGThreads = 512;

template <int DEC>
struct DecTraits;
template <> struct DecTraits<kDecVQ3> { static constexpr int bits = 6; };
template <> struct DecTraits<kDecLUT2> { static constexpr int bits = 2; };
template <> struct DecTraits<kDecLUT4> { static constexpr int bits = 4; };
template <> struct DecTraits<kDecDense> { static constexpr int bits = 16; };
template <> struct DecTraits<kDecVQ2> { static constexpr int bits = 4; };

template <int BM, int BN, int NMAT, int DEC, int EPI>
__global__ void __launch_bounds__(kGThreads, 1) k_gemm(GemmArgs a) {
    constexpr int LDK = kGK + kGPad;
    constexpr int WM = BM / 2, WN = BN / 4;   // per-wave outputs per matrix
    constexpr int TM = WM / 16, TN = WN / 16;  // 16x16 tiles per wave per matrix
    static_assert(TM >= 1 && TN >= 1, "tile too small");
    // One LDS block, the code tables first (address 0: a lookup address needs no base), then the
    // two activation and the two weight tile buffers.
    constexpr int kTabWords = DEC == kDecVQ3 ? 0 : DEC == kDecVQ2 ? NMAT * (BN / 8) * 16 : (BN / 8) * 8;
    constexpr int kOffX = (kTabWords * 4 + 255) / 256 * 256;
    constexpr int kOffW = kOffX + 2 * BM * LDK * 2;
    constexpr int kLds = kOffW + 2 * NMAT * BN * LDK * 2;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
    // VQ3: NMAT x (BN/8) groups x 64 dwords; LUT: (BN/8) x 16 halves
    uint32_t* const tabs = reinterpret_cast<uint32_t*>(lds);
    auto& Xs = *reinterpret_cast<uint16_t (*)[2][BM][LDK]>(lds + kOffX);
    auto& Ws = *reinterpret_cast<uint16_t (*)[2][NMAT][BN][LDK]>(lds + kOffW);

    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int N = a.N, K = a.K, T = a.T;
    const int KT = K / kGK;
    const int row0 = blockIdx.x * BN, tok0 = blockIdx.y * BM;
    const int ldo = a.ldo > 0 ? a.ldo : N;  // output row stride
    const int wm = w >> 2, wn = w & 3;

    // ---- tables.  VQ3: wave w decodes the GPW 8-row groups w * GPW .. (of all NMAT x BN/8) and
    // keeps each group's 64-entry codebook in one register (lane e holds entry e); a lookup is
    // a cross-lane read of that register (ds_bpermute), which never meets a bank conflict.
    constexpr int GPW = DEC == kDecVQ3 ? NMAT * BN / 64 : 1;  // groups per wave (8 waves)
    static_assert(DEC != kDecVQ3 || (NMAT * BN) % 64 == 0, "whole groups per wave");
    uint32_t cbr[GPW];
    if constexpr (DEC == kDecVQ3) {
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int G = w * GPW + i, m = G / (BN / 8), g = G % (BN / 8);
            const uint32_t* cb = (NMAT > 1 && m) ? a.cb[1] : a.cb[0];
            cbr[i] = cb[size_t(row0 / 8 + g) * 64 + l];
        }
    } else if constexpr (DEC == kDecLUT2 || DEC == kDecLUT4) {
        constexpr int E = 1 << DecTraits<DEC>::bits;
        const uint16_t* lut = reinterpret_cast<const uint16_t*>(a.cb[0]);
        uint16_t* t16 = reinterpret_cast<uint16_t*>(tabs);
        for (int i = tid; i < (BN / 8) * E; i += kGThreads)
            t16[(i / E) * 16 + (i % E)] = lut[size_t(row0 / 8) * E + i];
    } else if constexpr (DEC == kDecVQ2) {
        // group G = m * (BN / 8) + g: its 16 centroid words
        for (int i = tid; i < NMAT * (BN / 8) * 16; i += kGThreads) {
            const int G = i >> 4, m = G / (BN / 8), g = G % (BN / 8);
            const uint32_t* cb = (NMAT > 1 && m) ? a.cb[1] : a.cb[0];
            tabs[i] = cb[size_t(row0 / 8 + g) * 16 + (i & 15)];
        }
    }

    // ---- per-thread global fetch of one K tile
    // X: BM x 64 halves = BM*8 chunks of 16 bytes
    constexpr int XCH = BM * 8 / kGThreads;  // 16-byte chunks per thread
    u32x4 xr[2][XCH];  // two tiles in flight: the next one and the one after
    // weights: VQ3 -> NMAT*(BN/32) packed tiles x 64 lanes x 12 B (one lane record per thread);
    // LUT2 -> BN rows x 4 words (16 codes each); LUT4 -> BN rows x 8 words (2 per task);
    // DENSE -> BN rows x 64 halves (8 chunks of 16 B per row)
    constexpr int WTASKS = DEC == kDecVQ3 ? kGThreads * GPW  // one code record per group
                         : DEC == kDecLUT2 ? BN * 4
                         : DEC == kDecLUT4 ? BN * 4
                         : DEC == kDecVQ2  ? NMAT * BN  // (matrix, pair row, 32-column half)
                                           : BN * 8;
    constexpr int WPT = (WTASKS + kGThreads - 1) / kGThreads;
    constexpr int WW = DEC == kDecVQ3 ? 2 : DEC == kDecLUT2 ? 1 : DEC == kDecLUT4 ? 2 : 4;
    uint32_t wr[2][WPT][WW];  // raw words per task

    auto fetch = [&](int kt, int set) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + i * kGThreads;
            const int tt = c >> 3, c8 = (c & 7) * 8;
            const int tok = tok0 + tt;
            const uint16_t* src = a.x + size_t(tok < T ? tok : T - 1) * K + kt * kGK + c8;
            xr[set][i] = *reinterpret_cast<const u32x4*>(src);  // rows past T zeroed at stage
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int task = tid + i * kGThreads;
            if (task >= WTASKS) break;
            if constexpr (DEC == kDecVQ3) {
                // lane l decodes pair (l >> 4) of group G at columns 4 (l & 15) .. + 3: codes
                // 4 S .. 4 S + 3 (S = (l & 15) >> 2) of the packed lane record that holds
                // column group (l & 3) of the pair (record layout: see the skinny kernel)
                const int G = w * GPW + i, m = G / (BN / 8), g = G % (BN / 8);
                const int mt = row0 / 32 + g / 4, ll = ((l & 3) << 4) | (4 * (g % 4) + (l >> 4));
                // select between the two (uniform) base pointers instead of indexing the
                // argument array per lane, which would load the pointer and wait for it
                const uint8_t* cbase = (NMAT > 1 && m) ? a.codes[1] : a.codes[0];
                // the two record words that hold bits 24 S .. 24 S + 23: words 0, 1 for S < 2,
                // words 1, 2 otherwise
                const uint32_t* p = reinterpret_cast<const uint32_t*>(
                    cbase + (size_t(mt) * KT + kt) * kTileBytes) + 3 * ll + (((l & 15) >> 3) & 1);
                wr[set][i][0] = p[0];
                wr[set][i][1] = p[1];
            } else if constexpr (DEC == kDecVQ2) {
                // 32 codes (4 words) of pair row pr, columns 64 kt + 32 h ..
                const int m = task / BN, pr = (task % BN) >> 1, h = task & 1;
                const uint32_t* cbase = reinterpret_cast<const uint32_t*>((NMAT > 1 && m) ? a.codes[1] : a.codes[0]);
                const u32x4 v = *reinterpret_cast<const u32x4*>(
                    cbase + size_t(row0 / 2 + pr) * (K / 8) + kt * (kGK / 8) + 4 * h);
                wr[set][i][0] = v[0];
                wr[set][i][1] = v[1];
                wr[set][i][2] = v[2];
                wr[set][i][3] = v[3];
            } else if constexpr (DEC == kDecLUT2) {
                const int r = task >> 2, q = task & 3;  // 16 codes per word
                const uint32_t* p = reinterpret_cast<const uint32_t*>(a.codes[0]) +
                                    (size_t(row0 + r) * K + kt * kGK) / 16 + q;
                wr[set][i][0] = p[0];
            } else if constexpr (DEC == kDecLUT4) {
                const int r = task >> 2, q = task & 3;  // 2 words = 16 codes per task
                const uint32_t* p = reinterpret_cast<const uint32_t*>(a.codes[0]) +
                                    (size_t(row0 + r) * K + kt * kGK) / 8 + 2 * q;
                wr[set][i][0] = p[0];
                wr[set][i][1] = p[1];
            } else {
                const int r = task >> 3, c8 = (task & 7) * 8;
                const int row = row0 + r < N ? row0 + r : N - 1;
                const u32x4 v = *reinterpret_cast<const u32x4*>(a.dense + size_t(row) * K +
                                                                  kt * kGK + c8);
                wr[set][i][0] = v[0];
                wr[set][i][1] = v[1];
                wr[set][i][2] = v[2];
                wr[set][i][3] = v[3];
            }
        }
    };

    auto stage = [&](int buf, int set) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + i * kGThreads;
            const bool valid = tok0 + (c >> 3) < T;
            *reinterpret_cast<u32x4*>(&Xs[buf][c >> 3][(c & 7) * 8]) =
                valid ? xr[set][i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int task = tid + i * kGThreads;
            if (task >= WTASKS) break;
            if constexpr (DEC == kDecVQ3) {
                const int G = w * GPW + i, m = G / (BN / 8), g = G % (BN / 8);
                const int S = (l & 15) >> 2;
                // this lane's four codes: bits 24 S .. 24 S + 23 of the 96-bit record, from
                // its words (0, 1) when S < 2, else (1, 2)
                const uint32_t x = wr[set][i][0], y = wr[set][i][1];
                const uint32_t c4 = __builtin_amdgcn_alignbit(y, S == 3 ? y : x, (24 * S) & 31);
                uint32_t e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t addr = q ? (c4 >> (6 * q - 2)) & 0xFCu : (c4 << 2) & 0xFCu;
                    e[q] = uint32_t(__builtin_amdgcn_ds_bpermute(int(addr), int(cbr[i])));
                }
                // rows 2p, 2p + 1 of pair p = 4 g + (l >> 4), columns 4 (l & 15) .. + 3: each
                // 16-lane quarter writes one contiguous 128-byte row segment
                const int r = 8 * g + 2 * (l >> 4), c = 4 * (l & 15);
                *reinterpret_cast<u32x2*>(&Ws[buf][m][r][c]) =
                    u32x2{__builtin_amdgcn_perm(e[1], e[0], 0x05040100u),
                          __builtin_amdgcn_perm(e[3], e[2], 0x05040100u)};
                *reinterpret_cast<u32x2*>(&Ws[buf][m][r + 1][c]) =
                    u32x2{__builtin_amdgcn_perm(e[1], e[0], 0x07060302u),
                          __builtin_amdgcn_perm(e[3], e[2], 0x07060302u)};
            } else if constexpr (DEC == kDecVQ2) {
                // each code selects a centroid word: its low half goes to row 2 pr, its high half
                // to row 2 pr + 1, column 32 h + j
                const int m = task / BN, pr = (task % BN) >> 1, h = task & 1;
                const uint32_t* tg = tabs + (m * (BN / 8) + (pr >> 2)) * 16;
                uint32_t ev[16], od[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const uint32_t wv = wr[set][i][q >> 2];
                    const uint32_t c0 = (wv >> (8 * (q & 3))) & 15u, c1 = (wv >> (8 * (q & 3) + 4)) & 15u;
                    const uint32_t e0 = tg[c0], e1 = tg[c1];
                    ev[q] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
                    od[q] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
                }
                uint16_t* d0 = &Ws[buf][m][2 * pr][32 * h];
                uint16_t* d1 = &Ws[buf][m][2 * pr + 1][32 * h];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    *reinterpret_cast<u32x4*>(d0 + 8 * q) =
                        u32x4{ev[4 * q], ev[4 * q + 1], ev[4 * q + 2], ev[4 * q + 3]};
                    *reinterpret_cast<u32x4*>(d1 + 8 * q) =
                        u32x4{od[4 * q], od[4 * q + 1], od[4 * q + 2], od[4 * q + 3]};
                }
            } else if constexpr (DEC == kDecLUT2 || DEC == kDecLUT4) {
                constexpr int B = DecTraits<DEC>::bits;
                const int r = task >> 2, q = task & 3;
                const uint16_t* t16 = reinterpret_cast<const uint16_t*>(tabs) + (r >> 3) * 16;
                uint32_t out[8];
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    const int j0 = 2 * h, j1 = 2 * h + 1;  // code index within the 16
                    const uint32_t w0 = B == 2 ? wr[set][i][0] : wr[set][i][j0 >> 3];
                    const uint32_t w1 = B == 2 ? wr[set][i][0] : wr[set][i][j1 >> 3];
                    const uint32_t c0 = (w0 >> (B * (j0 & (32 / B - 1)))) & ((1u << B) - 1);
                    const uint32_t c1 = (w1 >> (B * (j1 & (32 / B - 1)))) & ((1u << B) - 1);
                    out[h] = uint32_t(t16[c0]) | (uint32_t(t16[c1]) << 16);
                }
                uint16_t* dst = &Ws[buf][0][r][16 * q];
                *reinterpret_cast<u32x4*>(dst) = u32x4{out[0], out[1], out[2], out[3]};
                *reinterpret_cast<u32x4*>(dst + 8) = u32x4{out[4], out[5], out[6], out[7]};
            } else {
                const int r = task >> 3, c8 = (task & 7) * 8;
                *reinterpret_cast<u32x4*>(&Ws[buf][0][r][c8]) =
                    u32x4{wr[set][i][0], wr[set][i][1], wr[set][i][2], wr[set][i][3]};
            }
        }
    };

    f32x4 acc[NMAT][TM][TN];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kGK / 32; ++ks) {
            const int kk = ks * 32 + 8 * (l >> 4);
            u32x4 A[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                A[i] = *reinterpret_cast<const u32x4*>(&Xs[buf][wm * WM + 16 * i + (l & 15)][kk]);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const u32x4 Bv =
                        *reinterpret_cast<const u32x4*>(&Ws[buf][m][wn * WN + 16 * j + (l & 15)][kk]);
#pragma unroll
                    for (int i = 0; i < TM; ++i) acc[m][i][j] = mfma16x16x32(A[i], Bv, acc[m][i][j]);
                }
        }
    };

    // Two raw tiles in flight in registers: tile kt + 2 is requested while tile kt is multiplied,
    // and decoded into LDS one step later, so its loads have two steps to arrive.
    // this workgroup's K tiles: split blockIdx.z of a.ksplit equal ranges
    const int nsplit = a.ksplit > 1 ? a.ksplit : 1;
    const int kb = int(blockIdx.z) * KT / nsplit, nk = (int(blockIdx.z) + 1) * KT / nsplit - kb;
    __syncthreads();  // tables
    fetch(kb, 0);
    fetch(kb + min(1, nk - 1), 1);
    stage(0, 0);
    __syncthreads();
    // The fetches are unconditional (tiles past the end reload the last one): a conditional
    // load would make the wait before each stage count no younger loads and drain the queue.
    // Each half-step stages unconditionally (past the end it decodes the clamped last tile into
    // a buffer nobody reads), so the products and the next tile's decode form one block of
    // independent instructions that the scheduler can interleave.
    for (int r = 0; r < nk; r += 2) {
        fetch(kb + min(r + 2, nk - 1), 0);
        compute(0);
        stage(1, 1);
        __syncthreads();
        if (r + 1 >= nk) break;
        fetch(kb + min(r + 3, nk - 1), 1);
        compute(1);
        stage(0, 0);
        __syncthreads();
    }

    // ---- epilogues.  Lane l, register r of tile (i, j) holds D[token][row] with
    // token = tok0 + wm*WM + 16 i + 4 (l/16) + r and row = row0 + wn*WN + 16 j + l%16.
    if constexpr (EPI == kEgLUT) {
        // scale, then add the rank-r product z U^T as one more K tile (z in X, U in W)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const float s = h2f(a.sc[0][row0 + wn * WN + 16 * j + (l & 15)]);
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[0][i][j] *= s;
        }
        for (int kr = 0; kr < a.r; kr += kGK) {
            for (int c = tid; c < BM * 8; c += kGThreads) {
                const int tt = c >> 3, c8 = (c & 7) * 8, tok = tok0 + tt;
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float z0 = 0.f, z1 = 0.f;
                    if (tok < T && kr + c8 + 2 * e < a.r) z0 = a.z[size_t(tok) * a.r + kr + c8 + 2 * e];
                    if (tok < T && kr + c8 + 2 * e + 1 < a.r) z1 = a.z[size_t(tok) * a.r + kr + c8 + 2 * e + 1];
                    h[e] = f2h(z0) | (f2h(z1) << 16);
                }
                *reinterpret_cast<u32x4*>(&Xs[0][tt][c8]) = u32x4{h[0], h[1], h[2], h[3]};
            }
            for (int c = tid; c < BN * 8; c += kGThreads) {
                const int rr = c >> 3, c8 = (c & 7) * 8;
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q0 = kr + c8 + 2 * e;
                    const uint32_t u0 = q0 < a.r ? a.U[size_t(row0 + rr) * a.r + q0] : 0u;
                    const uint32_t u1 = q0 + 1 < a.r ? a.U[size_t(row0 + rr) * a.r + q0 + 1] : 0u;
                    h[e] = u0 | (u1 << 16);
                }
                *reinterpret_cast<u32x4*>(&Ws[0][0][rr][c8]) = u32x4{h[0], h[1], h[2], h[3]};
            }
            __syncthreads();
            compute(0);
            __syncthreads();
        }
    }

    if constexpr (EPI == kEgGateUpRot) {
        // a = silu(g) u sign for BM tokens x BN (= one rotation block) rows, then the block
        // Hadamard transform along the rows in LDS (fp32, reusing the W buffers)
        static_assert(NMAT == 2, "gate+up");
        float* Ab = reinterpret_cast<float*>(lds + kOffX);  // [BM][BN + 1] over X and W
        static_assert(kLds - kOffX >= int(sizeof(float)) * BM * (BN + 1), "LDS for the rotation");
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int rl = wn * WN + 16 * j + (l & 15);
            const int row = row0 + rl;
            const float sg = h2f(a.sc[0][row]), su = h2f(a.sc[1][row]);
            const bool neg = a.sign && a.sign[row] < 0;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tl = wm * WM + 16 * i + 4 * (l >> 4) + r;
                    const float g = acc[0][i][j][r] * sg, u = acc[1][i][j][r] * su;
                    float v = silu(g) * u;
                    Ab[tl * (BN + 1) + rl] = neg ? -v : v;
                }
        }
        __syncthreads();
        for (int h = 1; h < BN; h <<= 1) {
            for (int i = tid; i < BM * (BN / 2); i += kGThreads) {
                const int tl = i / (BN / 2), jj = i % (BN / 2);
                const int lo = (jj / h) * 2 * h + (jj % h), hi = lo + h;
                const float x0 = Ab[tl * (BN + 1) + lo], x1 = Ab[tl * (BN + 1) + hi];
                Ab[tl * (BN + 1) + lo] = x0 + x1;
                Ab[tl * (BN + 1) + hi] = x0 - x1;
            }
            __syncthreads();
        }
        for (int i = tid; i < BM * BN / 2; i += kGThreads) {
            const int tl = i / (BN / 2), cc = (i % (BN / 2)) * 2;
            const int tok = tok0 + tl;
            if (tok < T) {
                const uint32_t h = f2h(Ab[tl * (BN + 1) + cc] * a.norm) |
                                   (f2h(Ab[tl * (BN + 1) + cc + 1] * a.norm) << 16);
                *reinterpret_cast<uint32_t*>(a.out16 + size_t(tok) * ldo + row0 + cc) = h;
            }
        }
        return;
    }

#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int row = row0 + wn * WN + 16 * j + (l & 15);
        if (row >= N) continue;
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
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = tok0 + wm * WM + 16 * i + 4 * (l >> 4) + r;
                if (tok >= T) continue;
                const float v0 = acc[0][i][j][r];
                if constexpr (EPI == kEgGateUp32) {
                    const float g = v0 * s0, u = acc[NMAT - 1][i][j][r] * s1;
                    const float act = silu(g) * u;
                    a.out32[size_t(tok) * ldo + row] = neg ? -act : act;
                } else if constexpr (EPI == kEgScale16 || EPI == kEgLUT) {
                    a.out16[size_t(tok) * ldo + row] = (uint16_t)f2h(v0 * s0);
                } else if constexpr (EPI == kEgPart2) {
                    // split z of a K-split gate/up product: unscaled g and u planes
                    float* o = a.out32 + (size_t(blockIdx.z) * T + tok) * 2 * N + row;
                    o[0] = v0;
                    o[N] = acc[NMAT - 1][i][j][r];
                } else {  // split z of a K-split product writes its own [T][N] plane
                    a.out32[(size_t(blockIdx.z) * T + tok) * N + row] = v0;
                }
            }
    }
}

template <int BM, int BN, int NMAT, int DEC, int EPI>
static hipError_t launch_gemm_t(const GemmArgs& a, hipStream_t st) {
    const dim3 grid((a.N + BN - 1) / BN, (a.T + BM - 1) / BM, a.ksplit > 1 ? a.ksplit : 1);
    hipLaunchKernelGGL((k_gemm<BM, BN, NMAT, DEC, EPI>), grid, dim3(kGThreads), 0, st, a);
    return hipGetLastError();
}

int gemm_split(int kind, int N, int K, int T, int cus) {
    // K splits that fill the CUs with whole rounds of workgroups where the output tiles alone
    // leave a partial last round.  The down projection keeps at least 8 K tiles per split
    // (the partial planes cost traffic); the small dense projection goes down to 2.
    const bool lut = kind == kGemmLUT2 || kind == kGemmLUT4;
    if ((kind != kGemmVQ3DownSplit && kind != kGemmDense32 && !lut) || T <= 0 || N <= 0 || cus <= 0)
        return 1;
    if (lut && T < kVq3mmMinT) return 1;
    const int kt = K / kGK;
    if ((kind == kGemmVQ3DownSplit || lut) && T >= kVq3mmMinT) {
        // whole rounds of workgroups, each extra plane priced at 1% of the product (the 64-row
        // prefill chunk's down projection: 10 splits of 20 tiles, 200 workgroups)
        const Vq3Tile t = vq3mm_tile(kind, T);
        const long tiles = long((N + t.bn - 1) / t.bn) * ((T + t.bm - 1) / t.bm);
        int best = 1;
        double best_cost = 1e9;
        for (int s = 1; s <= 16 && kt >= 4 * s; ++s) {
            const double cost = double((tiles * s + cus - 1) / cus) / s + 0.01 * (s - 1);
            if (cost < best_cost - 1e-9) {
                best = s;
                best_cost = cost;
            }
        }
        return best;
    }
    const int bm = T > 64 ? 128 : 64, bn = 64;
    const long tiles = long((N + bn - 1) / bn) * ((T + bm - 1) / bm);
    if (kind == kGemmDense32) {
        const long want = (2L * cus + tiles - 1) / tiles;
        return int(std::max(1L, std::min<long>(want, kt / 2)));
    }
    int best = 1;
    double best_waste = 1e9;
    for (int s = 1; s <= 16; s *= 2) {
        if (kt < 8 * s) break;
        const double rounds = double(tiles * s) / cus;
        const double waste = std::ceil(rounds) / rounds;
        if (waste < best_waste - 0.05) {
            best = s;
            best_waste = waste;
        }
    }
    return best;
}

// y = sc . (sum of the K-split planes), binary16.  Thread: V consecutive outputs (V = 4: 16-byte
// plane loads, N a multiple of 4), the planes' loads issued four at a time ahead of their sums; the
// sum of each output runs over the planes in order, whatever V.
template <int V>
__global__ void __launch_bounds__(256) k_split_reduce(int T, int N, int splits, const float* part,
                                                      const uint16_t* sc, uint16_t* y) {
    typedef float fv __attribute__((ext_vector_type(V)));
    const size_t n = size_t(T) * N;
    const size_t i = (size_t(blockIdx.x) * 256 + threadIdx.x) * V;
    if (i >= n) return;
    auto plane = [&](int z) { return *reinterpret_cast<const fv*>(part + size_t(z) * n + i); };
    fv sum = fv(0.f);
    int z = 0;
    for (; z + 4 <= splits; z += 4) {
        const fv p0 = plane(z), p1 = plane(z + 1), p2 = plane(z + 2), p3 = plane(z + 3);
        sum += p0;
        sum += p1;
        sum += p2;
        sum += p3;
    }
    for (; z < splits; ++z) sum += plane(z);
    const int row = int(i % size_t(N));
    uint32_t h[V];
#pragma unroll
    for (int e = 0; e < V; ++e) h[e] = f2h(sc ? sum[e] * h2f(sc[row + e]) : sum[e]);
    if constexpr (V == 4)  // 8-byte aligned (checked at launch)
        *reinterpret_cast<u32x2*>(y + i) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    else
        y[i] = uint16_t(h[0]);
}

hipError_t launch_split_reduce(int T, int N, int splits, const float* part, const uint16_t* sc,
                               uint16_t* y, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const size_t n = size_t(T) * N;
    if (N % 4 == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(y) & 7) == 0)
        hipLaunchKernelGGL(k_split_reduce<4>, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0, st,
                           T, N, splits, part, sc, y);
    else
        hipLaunchKernelGGL(k_split_reduce<1>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, T,
                           N, splits, part, sc, y);
    return hipGetLastError();
}

// out = sum of the planes (FP32).  A workgroup owns 32 outputs; its 8 thread groups sum
// interleaved subsets of the planes, then the 8 partial sums add in a fixed order.
__global__ void __launch_bounds__(256) k_split_sum(int n, int splits, const float* part,
                                                   float* out) {
    __shared__ float ps[8][32];
    const int o = threadIdx.x & 31, g = threadIdx.x >> 5, i = blockIdx.x * 32 + o;
    float sum = 0.f;
    if (i < n)
        for (int z = g; z < splits; z += 8) sum += part[size_t(z) * n + i];
    ps[g][o] = sum;
    __syncthreads();
    if (g == 0 && i < n) {
        float v = ps[0][o];
#pragma unroll
        for (int k = 1; k < 8; ++k) v += ps[k][o];
        out[i] = v;
    }
}

hipError_t launch_split_sum(int n, int splits, const float* part, float* out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_split_sum, dim3((n + 31) / 32), dim3(256), 0, st, n, splits, part, out);
    return hipGetLastError();
}

// Finish a K-split gate/up product: a = silu(sc_g . sum g) . (sc_u . sum u) . sign for rows
// [0, N) of the split part, then either the 128-wide rotation (binary16 out) or FP32 out.
// One wave per (token, 128-row block); value e of lane l is row 64 e + l of the block.
__global__ void __launch_bounds__(256) k_gateup_combine(int T, int N, int splits,
                                                        const float* part, const uint16_t* scg,
                                                        const uint16_t* scu, const int8_t* sign,
                                                        int rotate, float norm, int ldo,
                                                        uint16_t* out16, float* out32) {
    const int l = threadIdx.x & 63, wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nb = N / 128;
    if (wv >= T * nb) return;
    const int t = wv / nb, r0 = (wv % nb) * 128;
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int row = r0 + 64 * e + l;
        // the planes' loads four at a time ahead of their sums, each sum over the planes in order
        const float* p = part + size_t(t) * 2 * N + row;
        const size_t zs = size_t(T) * 2 * N;  // plane stride
        float g = 0.f, u = 0.f;
        int z = 0;
        for (; z + 4 <= splits; z += 4) {
            float pg[4], pu[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                pg[k] = p[(z + k) * zs];
                pu[k] = p[(z + k) * zs + N];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                g += pg[k];
                u += pu[k];
            }
        }
        for (; z < splits; ++z) {
            g += p[z * zs];
            u += p[z * zs + N];
        }
        g *= h2f(scg[row]);
        u *= h2f(scu[row]);
        const float act = silu(g) * u;
        v[e] = sign && sign[row] < 0 ? -act : act;
    }
    if (!rotate) {
#pragma unroll
        for (int e = 0; e < 2; ++e) out32[size_t(t) * ldo + r0 + 64 * e + l] = v[e];
        return;
    }
    for (int h = 1; h < 64; h <<= 1) {
        const bool upper = (l & h) != 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float p = __shfl_xor(v[e], h);
            v[e] = upper ? p - v[e] : v[e] + p;
        }
    }
    const float x0 = v[0], x1 = v[1];
    v[0] = x0 + x1;
    v[1] = x0 - x1;
#pragma unroll
    for (int e = 0; e < 2; ++e)
        out16[size_t(t) * ldo + r0 + 64 * e + l] = (uint16_t)f2h(v[e] * norm);
}

hipError_t launch_gateup_combine(int T, int N, int splits, const float* part,
                                 const uint16_t* scg, const uint16_t* scu, const int8_t* sign,
                                 int rotate, float norm, int ldo, uint16_t* out16, float* out32,
                                 hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (N % 128) return hipErrorInvalidValue;
    const int waves = T * (N / 128);
    hipLaunchKernelGGL(k_gateup_combine, dim3((waves + 3) / 4), dim3(256), 0, st, T, N, splits,
                       part, scg, scu, sign, rotate, norm, ldo, out16, out32);
    return hipGetLastError();
}

// The VQ3 kinds on 2x16 matrices: the tiled kernels with the 2x16 decoder at every T.
static hipError_t launch_gemm_vq2(const GemmArgs& a, hipStream_t st) {
    if (a.K % kGK || a.N <= 0 || a.N % 64) return hipErrorInvalidValue;
    if (a.ksplit > 1 && (a.kind != kGemmVQ3DownSplit && a.kind != kGemmVQ3GateUpSplit))
        return hipErrorInvalidValue;
    if (a.ksplit > 1 && (a.K / kGK) < a.ksplit) return hipErrorInvalidValue;
    const bool big = a.T > 64, n128 = a.N % 128 == 0;
    switch (a.kind) {
        case kGemmVQ3GateUp:
            if (n128)
                return big ? launch_gemm_t<128, 128, 2, kDecVQ2, kEgGateUp32>(a, st)
                           : launch_gemm_t<64, 128, 2, kDecVQ2, kEgGateUp32>(a, st);
            return big ? launch_gemm_t<128, 64, 2, kDecVQ2, kEgGateUp32>(a, st)
                       : launch_gemm_t<64, 64, 2, kDecVQ2, kEgGateUp32>(a, st);
        case kGemmVQ3GateUpRot:
            if (!n128) return hipErrorInvalidValue;
            return big ? launch_gemm_t<128, 128, 2, kDecVQ2, kEgGateUpRot>(a, st)
                       : launch_gemm_t<64, 128, 2, kDecVQ2, kEgGateUpRot>(a, st);
        case kGemmVQ3Down:
            return big ? launch_gemm_t<128, 64, 1, kDecVQ2, kEgScale16>(a, st)
                       : launch_gemm_t<64, 64, 1, kDecVQ2, kEgScale16>(a, st);
        case kGemmVQ3DownSplit:
            return big ? launch_gemm_t<128, 64, 1, kDecVQ2, kEgPlain32>(a, st)
                       : launch_gemm_t<64, 64, 1, kDecVQ2, kEgPlain32>(a, st);
        case kGemmVQ3GateUpSplit:
            if (!n128) return hipErrorInvalidValue;
            return big ? launch_gemm_t<128, 128, 2, kDecVQ2, kEgPart2>(a, st)
                       : launch_gemm_t<64, 128, 2, kDecVQ2, kEgPart2>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.vq2 && a.T < kVq3mmMinT) return launch_gemm_vq2(a, st);
    if (a.T >= kVq3mmMinT &&
        (a.kind == kGemmVQ3GateUp || a.kind == kGemmVQ3GateUpRot || a.kind == kGemmVQ3Down ||
         a.kind == kGemmVQ3GateUpSplit || a.kind == kGemmVQ3DownSplit || a.kind == kGemmLUT2 ||
         a.kind == kGemmLUT4))
        return launch_vq3mm(a, st);
    if (a.K % kGK || a.N <= 0) return hipErrorInvalidValue;
    if (a.ksplit > 1 && ((a.kind != kGemmVQ3DownSplit && a.kind != kGemmDense32 &&
                          a.kind != kGemmVQ3GateUpSplit) ||
                         (a.K / kGK) < a.ksplit))
        return hipErrorInvalidValue;
    // only the dense decoder clamps its rows; the coded ones need whole 64-row tiles
    if (a.kind != kGemmDense32 && a.N % 64) return hipErrorInvalidValue;
    const bool big = a.T > 64;          // 128-token tiles beyond one 64-row chunk
    const bool n128 = a.N % 128 == 0;   // 128-row tiles where the rows allow it
#define VQ_BM_BN(NM, DEC, EPI)                                                              \
    (big ? (n128 ? launch_gemm_t<128, 128, NM, DEC, EPI>(a, st)                             \
                 : launch_gemm_t<128, 64, NM, DEC, EPI>(a, st))                             \
         : (n128 ? launch_gemm_t<64, 128, NM, DEC, EPI>(a, st)                              \
                 : launch_gemm_t<64, 64, NM, DEC, EPI>(a, st)))
    switch (a.kind) {
        case kGemmVQ3GateUp:
            return VQ_BM_BN(2, kDecVQ3, kEgGateUp32);
        case kGemmVQ3GateUpRot:  // the rotation block is the 128-row tile
            if (!n128) return hipErrorInvalidValue;
            return big ? launch_gemm_t<128, 128, 2, kDecVQ3, kEgGateUpRot>(a, st)
                       : launch_gemm_t<64, 128, 2, kDecVQ3, kEgGateUpRot>(a, st);
        case kGemmVQ3Down:  // 64-row tiles: the down projection has few rows
            return big ? launch_gemm_t<128, 64, 1, kDecVQ3, kEgScale16>(a, st)
                       : launch_gemm_t<64, 64, 1, kDecVQ3, kEgScale16>(a, st);
        case kGemmLUT2:
            return VQ_BM_BN(1, kDecLUT2, kEgLUT);
        case kGemmLUT4:
            return VQ_BM_BN(1, kDecLUT4, kEgLUT);
        case kGemmDense32:
            return big ? launch_gemm_t<128, 64, 1, kDecDense, kEgPlain32>(a, st)
                       : launch_gemm_t<64, 64, 1, kDecDense, kEgPlain32>(a, st);
        case kGemmVQ3GateUpSplit:  // unscaled g and u planes, one pair per K split
            if (!n128) return hipErrorInvalidValue;
            return big ? launch_gemm_t<128, 128, 2, kDecVQ3, kEgPart2>(a, st)
                       : launch_gemm_t<64, 128, 2, kDecVQ3, kEgPart2>(a, st);
        case kGemmVQ3DownSplit:  // unscaled FP32 partial sums, one plane per K split
            return big ? launch_gemm_t<128, 64, 1, kDecVQ3, kEgPlain32>(a, st)
                       : launch_gemm_t<64, 64, 1, kDecVQ3, kEgPlain32>(a, st);
    }
#undef VQ_BM_BN
    return hipErrorInvalidValue;
}

}  // namespace vqmlp
