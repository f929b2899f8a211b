// vq3mm.hip -- matrix-core product with the VQ3 weights decoded in registers, for T > 32 rows
// (gfx950).
//
//   D[t][n] = sum_k X[t][k] W[n][k],   X binary16 [T][K] (rotated activations), W packed VQ3.
//
// Model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP, token-mixer
// rotations, distilled weights": a six-bit code selects the pair (W[2p][j], W[2p+1][j]) from 64
// two-component binary16 centroids shared by 8 rows; row scales are applied in the epilogue.
// The same kernel serves the 2x16 format (4-bit codes, 16 centroids) and the scalar-LUT
// projections (2- or 4-bit codes into per-8-row tables of scalars).
//
// Work split.  A workgroup of NW waves owns BM tokens x NW*RW rows (of each of NMAT matrices
// that share X).  Each wave owns RW rows and all BM tokens, so no weight is used by two waves and
// the decoded weights never pass through LDS: a wave turns its own codes straight into the B
// operands of v_mfma_f32_32x32x16_f16.  Only the activation tile is staged through LDS, where
// all waves read it.  NW = 4 is one wave per SIMD (accumulators in the AGPRs); from 256 tokens the
// VQ kinds run NW = 8, two waves per SIMD, so that one wave decodes while the other multiplies.
//
// Decoding.  A B operand is 32 rows x 16 K columns.  The centroids of its four 8-row groups sit
// in one LDS table replicated over the 32 bank columns (column b holds group b / 8), and lane l,
// whose row is l % 32, reads column l % 32 only: a lookup is one 4-byte LDS read at (code, own
// column), free of bank conflicts whatever the codes.  A centroid holds both rows of a pair, so a
// lane fetches its pair's centroids for four of its eight columns, keeps its own row's halves and
// trades the other halves with lane l ^ 1 (one DPP quad permute).  The tables are written once
// per workgroup: the codebooks are shared by all K.
//
// Codes and activations.  The codes a lane needs for one 64-column K tile (four K steps) are one
// 96-bit lane record of the packed tile, 24 bits per K step.  The activations are staged into LDS
// with 16-byte chunks XOR-swizzled by row, so an A operand is one conflict-free 16-byte read.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace vqmlp {

namespace {

constexpr int kXK = 64;   // K tile

constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3: 32-bit raw data
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2] -- lane n reads lane n ^ 1

__device__ __forceinline__ uint32_t from_xor1(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), kDppXor1, 0xF, 0xF, false));
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

template <int NW, int BM, int RW, int NMAT, int DEC, int EPI, int CQ>
__global__ void __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
k_vq3mm(GemmArgs a) {
    constexpr bool VQ = DEC == kDecVQ3;
    constexpr bool V2 = DEC == kDecVQ2;  // 2x16: 4-bit codes into 16 centroids per 8 rows
    constexpr bool PAIR = VQ || V2;      // a centroid holds both rows of a pair
    constexpr int BITS = DEC == kDecLUT2 ? 2 : 4;  // scalar-LUT code width
    constexpr int NT = NW * 64;
    constexpr int RF = RW / 32;       // 32-row B operands per wave per matrix
    constexpr int TF = BM / 32;       // 32-token A operands
    constexpr int BNW = NW * RW;      // rows per workgroup
    constexpr int NB = NMAT * RF;     // B operands per K step (one centroid table each)
    constexpr int XCH = BM * 8 / NT;  // 16-byte activation chunks per thread per K tile
    static_assert(RW % 32 == 0 && XCH >= 1 && (BM * 8) % NT == 0, "shape");
    constexpr int kEnt = VQ ? 64 : 16;           // table entries
    constexpr int kTabBytes = kEnt * 32 * 4;     // entries x 32 bank columns
    constexpr int kOffX = NW * NB * kTabBytes;  // activation tiles after the tables
    constexpr int kXBuf = BM * kXK * 2;         // one activation tile
    constexpr int kMain = kOffX + 2 * kXBuf;
    constexpr int kEpBytes = EPI == kEgGateUpRot ? BM * (BNW + 1) * 4 : 0;
    static_assert(PAIR || (NMAT == 1 && (EPI == kEgLUT || EPI == kEgLUTPlane)), "LUT: one matrix");
    constexpr int kLds = kMain > kEpBytes ? kMain : kEpBytes;
    static_assert(kLds <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];

    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int n = l & 31, kh = l >> 5, c0 = n & 1, pr = n >> 1;
    const int N = a.N, K = a.K, T = a.T, KT = K / kXK;
    const int row0 = blockIdx.x * BNW, tok0 = blockIdx.y * BM;
    const int wrow = row0 + w * RW;  // first row of this wave
    const int ldo = a.ldo > 0 ? a.ldo : N;
    const int mt_last = N / 32 - 1;

    // ---- lookup tables.  Table (m, j) serves B operand j of matrix m (rows wrow + 32 j ..,
    // four 8-row groups): word (e, b) -- entry e, bank column b -- holds entry e of group b / 8.
    // Lane l reads column l % 32 only, which holds its own row's group, so a lookup never meets a
    // bank conflict.  Entries: VQ3, the 64 two-component centroids; 2x16, the 16 two-component
    // centroids; LUT2, the 16 pairs (lut[e % 4], lut[e / 4]) of two neighbouring codes; LUT4, the
    // 16 scalars (low half).
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const uint32_t* cb = (NMAT > 1 && m) ? a.cb[1] : a.cb[0];
        const uint16_t* lut = reinterpret_cast<const uint16_t*>(a.cb[0]);
#pragma unroll
        for (int j = 0; j < RF; ++j) {
            unsigned char* tb = lds + (w * NB + m * RF + j) * kTabBytes;
            const int g0 = wrow / 8 + 4 * j;
#pragma unroll
            for (int k = 0; k < kEnt * 8 / 64; ++k) {
                const int idx = l + 64 * k, e = idx >> 3, bq = idx & 7;  // 4 columns per store
                const int grp = min(g0 + (bq >> 1), N / 8 - 1);
                uint32_t v;
                if constexpr (VQ)
                    v = cb[size_t(grp) * 64 + e];
                else if constexpr (V2)
                    v = cb[size_t(grp) * 16 + e];
                else if constexpr (DEC == kDecLUT2)
                    v = uint32_t(lut[size_t(grp) * 4 + (e & 3)]) | (uint32_t(lut[size_t(grp) * 4 + (e >> 2)]) << 16);
                else
                    v = lut[size_t(grp) * 16 + e];
                *reinterpret_cast<u32x4*>(tb + e * 128 + bq * 16) = u32x4{v, v, v, v};
            }
        }
    }
    const uint32_t tab_lane = uint32_t(w * NB * kTabBytes) + uint32_t(n) * 4u;

    // ---- this lane's codes.  Lane l holds B rows n = l % 32 (pair pr, component c0) at K
    // columns 16 ks + 8 kh .. + 7 of each 16-column K step ks.  It looks up its pair's centroids
    // for columns 4 c0 .. 4 c0 + 3 of those eight: for all four K steps these are the 16 codes of
    // lane record (2 kh + c0, pair) of the packed tile, K step ks in its 24-bit slot ks.
    // 2x16 codes are packed by pair row, 8 columns per word.  Their K steps take the columns of
    // a tile in another order (below), in which the lane's 16 codes of a tile are the two words
    // 4 c0 + 2 kh and 4 c0 + 2 kh + 1 of its pair row: K step ks in half ks % 2 of word ks / 2.
    // Scalar LUTs are packed row by row (32 / BITS codes per word, low bits first): a K tile is
    // 8 BITS bytes of each row, K step ks in word ks (LUT2, half kh) or word 2 ks + kh (LUT4).
    constexpr int CW = VQ ? 3 : V2 ? 2 : 2 * BITS;  // code words per lane per operand and K tile
    constexpr int kTileCode = VQ ? kTileBytes : V2 ? 32 : 8 * BITS;  // bytes per K tile
    uint32_t voff[RF];
#pragma unroll
    for (int j = 0; j < RF; ++j) {
        if constexpr (VQ) {
            const int mt = min(wrow / 32 + j, mt_last);
            voff[j] = uint32_t(mt) * uint32_t(KT) * kTileBytes +
                      12u * uint32_t(((2 * kh + c0) << 4) | pr);
        } else if constexpr (V2) {
            const int pair = min((wrow + 32 * j) / 2 + pr, N / 2 - 1);
            voff[j] = uint32_t(pair) * uint32_t(K / 2) + 4u * uint32_t(4 * c0 + 2 * kh);
        } else {
            const int row = min(wrow + 32 * j + n, N - 1);
            voff[j] = uint32_t(row) * uint32_t(K / 8 * BITS);
        }
    }
    // v_perm selectors: this lane's component and the partner's
    const uint32_t sel_own = c0 ? 0x07060302u : 0x05040100u;
    const uint32_t sel_oth = c0 ? 0x05040100u : 0x07060302u;

    // ---- activation tiles in LDS: row r (token), 16-byte chunk q (columns 8q .. 8q + 7) stored
    // at chunk q ^ (r % 8), so that the eight rows read together hit eight different chunks.
    uint32_t aoff[4];  // A operand of K step ks: row n, chunk 2 ks + kh
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        aoff[ks] = kOffX + uint32_t(n) * 128u + (uint32_t((2 * ks + kh) ^ (n & 7)) << 4);
    // staging: chunk x of this thread is token row tid / 8 + x NT / 8, columns 8 (tid % 8) ..;
    // all of a thread's chunks share row % 8, hence one address plus constant offsets
    static_assert((NT / 8) % 8 == 0, "chunks of one thread share the row swizzle");
    const uint32_t xw = kOffX + uint32_t(tid >> 3) * 128u + (uint32_t((tid & 7) ^ ((tid >> 3) & 7)) << 4);
    // 2x16 column order: slot (ks, kh, i) of the A and B operands is column 32 (i / 4) + 16 kh +
    // 4 ks + i % 4 of the tile, so that half h of the thread's chunk q (columns 8 q + 4 h ..) goes
    // to 8 bytes 8 (q / 4) of 16-byte chunk 2 ks + kh, ks = (2 q + h) % 4, kh = (q / 2) % 2
    uint32_t xw2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = tid & 7, c = 2 * ((2 * q + h) & 3) + ((q >> 1) & 1);
        xw2[h] = kOffX + uint32_t(tid >> 3) * 128u + (uint32_t(c ^ ((tid >> 3) & 7)) << 4) + 8u * uint32_t(q >> 2);
    }
    uint32_t xoff[XCH];  // global byte offset of the chunk in K tile 0
#pragma unroll
    for (int x = 0; x < XCH; ++x) {
        const int c = tid + x * NT;
        // rows past T repeat row T - 1: their products are never stored
        const int tok = min(tok0 + (c >> 3), T - 1);
        xoff[x] = (uint32_t(tok) * uint32_t(K) + 8u * uint32_t(c & 7)) * 2u;
    }

    // Loads go through buffer resources: the lane's offset is fixed for the whole K loop and the
    // K tile's offset rides in the scalar offset, so no address arithmetic is spent per load.
    __amdgpu_buffer_rsrc_t rs_code[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        rs_code[m] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>((NMAT > 1 && m) ? a.codes[1] : a.codes[0]), 0,
            int(VQ   ? uint32_t(N / 32) * uint32_t(KT) * kTileBytes
                : V2 ? uint32_t(N / 2) * uint32_t(K / 2)
                     : uint32_t(N) * uint32_t(K / 8 * BITS)),
            kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x), 0, int(uint32_t(T) * uint32_t(K) * 2u), kRsrcWord3);

    u32x4 xr[XCH];            // activation chunks of the next K tile
    // code words of the next CQ K tiles: tile t lives in slot t % CQ, requested CQ tiles before
    // the products reach it (the K loop is unrolled by CQ so every slot index is a constant)
    uint32_t rn[CQ][NMAT][RF][CW];
    uint32_t rc[NMAT][RF][CW];  // code words being decoded
    u32x4 Bf[4][NMAT][RF];    // B operands [ks][m][j]

    auto load_x = [&](int kt) {
#pragma unroll
        for (int x = 0; x < XCH; ++x)
            xr[x] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, int(xoff[x]), kt * kXK * 2, 0));
    };
    auto load_codes = [&](int kt, int slot) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j) {
                if constexpr (VQ) {
                    const u32x3 v = __builtin_bit_cast(
                        u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs_code[m], int(voff[j]),
                                                                    kt * kTileCode, 0));
#pragma unroll
                    for (int q = 0; q < 3; ++q) rn[slot][m][j][q] = v[q];
                } else if constexpr (V2) {
                    const u32x2 v = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs_code[m], int(voff[j]),
                                                                    kt * kTileCode, 0));
                    rn[slot][m][j][0] = v[0];
                    rn[slot][m][j][1] = v[1];
                } else {
#pragma unroll
                    for (int h = 0; h < CW / 4; ++h) {
                        const u32x4 v = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rs_code[m], int(voff[j]) + 16 * h, kt * kTileCode, 0));
#pragma unroll
                        for (int q = 0; q < 4; ++q) rn[slot][m][j][4 * h + q] = v[q];
                    }
                }
            }
    };
    auto stage = [&](uint32_t bufoff) {
        if constexpr (V2) {
#pragma unroll
            for (int x = 0; x < XCH; ++x) {
                *reinterpret_cast<u32x2*>(lds + xw2[0] + bufoff + x * (NT / 8) * 128) = u32x2{xr[x][0], xr[x][1]};
                *reinterpret_cast<u32x2*>(lds + xw2[1] + bufoff + x * (NT / 8) * 128) = u32x2{xr[x][2], xr[x][3]};
            }
        } else {
            unsigned char* base = lds + (xw + bufoff);
#pragma unroll
            for (int x = 0; x < XCH; ++x)
                *reinterpret_cast<u32x4*>(base + x * (NT / 8) * 128) = xr[x];
        }
    };
    auto take_codes = [&](int slot) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j)
#pragma unroll
                for (int q = 0; q < CW; ++q) rc[m][j][q] = rn[slot][m][j][q];
    };

    // Decoding B operand (ks, b = (m, j)), in two phases: the four table reads (centroids of the
    // lane's pair at its four columns), then the exchange with lane l ^ 1 that gives each lane its
    // own row's halves at all eight columns.
    constexpr int NE = DEC == kDecLUT4 ? 8 : 4;  // table reads per operand and K step
    uint32_t ev[2][NE];                          // table reads of two operands in flight
    auto dec_read = [&](int ks, int b) {
        const int m = b / RF, j = b % RF;
        const unsigned char* tb = lds + b * kTabBytes;
        if constexpr (VQ) {
            const uint32_t* r = rc[m][j];
            // code k of K step ks at record bit 24 ks + 6 k, moved to bits 12:7
            uint32_t x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int bit = 24 * ks + 6 * k;
                const int wd = bit / 32, sh = bit % 32;
                if (sh <= 7)
                    x[k] = r[wd] << (7 - sh);
                else if (sh <= 26)
                    x[k] = r[wd] >> (sh - 7);
                else
                    x[k] = __builtin_amdgcn_alignbit(r[wd + 1], r[wd], sh - 7);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                ev[b & 1][k] = *reinterpret_cast<const uint32_t*>(tb + and_or(x[k], 0x1F80u, tab_lane));
        } else if constexpr (V2) {
            // the lane's 16 bits of K step ks: code k (4 bits) at bit 4 k, moved to bits 10:7
            const uint32_t wk = rc[m][j][ks >> 1] >> (16 * (ks & 1));
            const uint32_t x[4] = {wk << 7, wk << 3, wk >> 1, wk >> 5};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                ev[b & 1][k] = *reinterpret_cast<const uint32_t*>(tb + and_or(x[k], 0x780u, tab_lane));
        } else if constexpr (DEC == kDecLUT2) {
            // the lane's 16 bits of word ks: code pair p (4 bits) at bit 4 p, moved to bits 10:7
            const uint32_t wk = rc[m][j][ks] >> (16 * kh);
            const uint32_t x[4] = {wk << 7, wk << 3, wk >> 1, wk >> 5};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                ev[b & 1][k] = *reinterpret_cast<const uint32_t*>(tb + and_or(x[k], 0x780u, tab_lane));
        } else {
            // word 2 ks + kh: code i (4 bits) at bit 4 i, moved to bits 10:7
            const uint32_t wd = kh ? rc[m][j][2 * ks + 1] : rc[m][j][2 * ks];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t x = i < 2 ? wd << (7 - 4 * i) : wd >> (4 * i - 7);
                ev[b & 1][i] = *reinterpret_cast<const uint16_t*>(tb + and_or(x, 0x780u, tab_lane));
            }
        }
    };
    auto dec_place = [&](int ks, int b) {
        const int m = b / RF, j = b % RF;
        if constexpr (DEC == kDecLUT2) {
            Bf[ks][m][j] = u32x4{ev[b & 1][0], ev[b & 1][1], ev[b & 1][2], ev[b & 1][3]};
            return;
        } else if constexpr (DEC == kDecLUT4) {
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = ev[b & 1][2 * q] | (ev[b & 1][2 * q + 1] << 16);
            Bf[ks][m][j] = v;
            return;
        }
        const uint32_t e0 = ev[b & 1][0], e1 = ev[b & 1][1], e2 = ev[b & 1][2], e3 = ev[b & 1][3];
        const uint32_t y0 = __builtin_amdgcn_perm(e1, e0, sel_own);
        const uint32_t y1 = __builtin_amdgcn_perm(e3, e2, sel_own);
        const uint32_t r0 = from_xor1(__builtin_amdgcn_perm(e1, e0, sel_oth));
        const uint32_t r1 = from_xor1(__builtin_amdgcn_perm(e3, e2, sel_oth));
        Bf[ks][m][j] = c0 ? u32x4{r0, r1, y0, y1} : u32x4{y0, y1, r0, r1};
    };

    f32x16 acc[NMAT][RF][TF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < RF; ++j)
#pragma unroll
            for (int i = 0; i < TF; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[m][j][i][q] = 0.f;

    auto readA = [&](uint32_t bufoff, int ks, int i) {
        return *reinterpret_cast<const u32x4*>(lds + aoff[ks] + bufoff + i * 32 * 128);
    };
    auto mma_unit = [&](int ks, int i, const u32x4& A) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j) acc[m][j][i] = mfma32x32x16(A, Bf[ks][m][j], acc[m][j][i]);
    };

    // this workgroup's K tiles: split blockIdx.z of a.ksplit equal ranges
    const int nsplit = a.ksplit > 1 ? a.ksplit : 1;
    const int kb = int(blockIdx.z) * KT / nsplit, nk = (int(blockIdx.z) + 1) * KT / nsplit - kb;
    auto tile = [&](int t) { return kb + min(t, nk - 1); };  // loads past the end repeat the last

    // Prologue: tables, tile 0's activations in buffer 0, its K steps 0 and 1 decoded; the codes
    // of tiles 1 .. CQ and the activations of tile 1 requested.
    load_codes(tile(0), 0);
    load_x(tile(0));
    __syncthreads();  // tables
    take_codes(0);
#pragma unroll
    for (int q = 1; q <= CQ; ++q) load_codes(tile(q), q % CQ);
    stage(0);
    load_x(tile(1));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            dec_read(ks, b);
            dec_place(ks, b);
        }
    __syncthreads();

    // One K tile per iteration, hand-interleaved.  The products of tile t run in 4 TF units (one
    // A operand, NB matrix-core steps each): those of K steps 0 and 1 beside the decoding of the
    // tile's K steps 2 and 3, those of K steps 2 and 3 beside the decoding of tile t + 1's K steps
    // 0 and 1, each into the registers its products have just released.  Mid-tile the code
    // records of tile t + 1 are taken and tile t + 2's requested; at the end tile t + 1's
    // activations are staged and tile t + 2's requested.  A operands are read two units ahead;
    // scheduling barriers keep this order.  Every load is unconditional, so each wait counts the
    // same loads on every path.
    constexpr int MU = 4 * TF;  // product units per K tile
    constexpr int DU = 4 * NB;  // decoded operands per K tile
    static_assert(MU % DU == 0 && MU / DU >= 1, "whole product units per decoded operand");
    constexpr int PER = MU / DU;
    for (int t0 = 0; t0 < nk; t0 += CQ)
#pragma unroll
    for (int tu = 0; tu < CQ; ++tu) {
        const int t = t0 + tu;
        if (t >= nk) break;
        const int slot = (tu + 1) % CQ;  // holds tile t + 1 (t0 is a multiple of CQ)
        const uint32_t cur = uint32_t(t & 1) * kXBuf, nxt = uint32_t(kXBuf) - cur;
        u32x4 Ar[3];
        Ar[0] = readA(cur, 0, 0);
        Ar[1] = readA(cur, 0, 1 % TF);
        dec_read(2, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < MU; ++c) {
            const int ks = c / TF, i = c % TF;
            if (c + 2 < MU) Ar[(c + 2) % 3] = readA(cur, (c + 2) / TF, (c + 2) % TF);
            mma_unit(ks, i, Ar[c % 3]);
            // decoded operand d = c / PER of this tile's list: K steps 2, 3 of tile t, then K
            // steps 0, 1 of tile t + 1 (its codes taken once the list reaches them)
            if (c % PER == PER - 1 || PER == 1) {
                const int d = c / PER;
                const int dks = (d / NB + 2) % 4, db = d % NB;
                dec_place(dks, db);
                if (d + 1 < DU) {
                    const int nks = ((d + 1) / NB + 2) % 4, nb = (d + 1) % NB;
                    if (d + 1 == 2 * NB) {  // tile t's records are read: take tile t + 1's
                        take_codes(slot);
                        load_codes(tile(t + 1 + CQ), slot);
                    }
                    dec_read(nks, nb);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        stage(nxt);  // activations of tile t + 1
        load_x(tile(t + 2));
        __syncthreads();
    }
    if constexpr (EPI == kEgGateUpRot) __syncthreads();  // the epilogue reuses the LDS

    // ---- epilogues.  Lane l, register q of acc[m][j][i] holds D[token][row] with
    // token = tok0 + 32 i + 8 (q / 4) + 4 kh + q % 4 and row = wrow + 32 j + n.
    if constexpr (EPI == kEgGateUpRot) {
        // a = silu(g) u sign over BM tokens x BNW rows in LDS (fp32), then the Hadamard transform
        // of every 128-row block, then binary16 out
        static_assert(NMAT == 2 && BNW % 128 == 0, "gate+up, whole rotation blocks");
        float* Ab = reinterpret_cast<float*>(lds);  // [BM][BNW + 1]
#pragma unroll
        for (int j = 0; j < RF; ++j) {
            const int rl = w * RW + 32 * j + n;
            const int row = min(row0 + rl, N - 1);
            const float sg = h2f(a.sc[0][row]), su = h2f(a.sc[1][row]);
            const bool neg = a.sign && a.sign[row] < 0;
#pragma unroll
            for (int i = 0; i < TF; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int tl = 32 * i + 8 * (q >> 2) + 4 * kh + (q & 3);
                    const float g = acc[0][j][i][q] * sg, u = acc[1][j][i][q] * su;
                    const float v = silu(g) * u;
                    Ab[tl * (BNW + 1) + rl] = neg ? -v : v;
                }
        }
        __syncthreads();
        // The butterflies of distance 1, 2, 4, then of 8, 16, 32, three stages per LDS pass on 8
        // values in registers (thread: one token and 8 rows h apart; consecutive threads take
        // consecutive tokens, whose rows lie one bank apart in the padded layout); the stage of
        // distance 64 runs in the binary16 stores.  Every value meets the same additions in the
        // same order as with one pass per stage.
        auto radix8 = [&](const int h) {
            for (int e = tid; e < BM * (BNW / 8); e += NT) {
                const int tl = e % BM, jj = e / BM;
                float* p = Ab + tl * (BNW + 1) + (jj / h) * 8 * h + (jj % h);
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = p[k * h];
#pragma unroll
                for (int d = 1; d < 8; d <<= 1)
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (!(k & d)) {
                            const float x0 = v[k], x1 = v[k | d];
                            v[k] = x0 + x1;
                            v[k | d] = x0 - x1;
                        }
#pragma unroll
                for (int k = 0; k < 8; ++k) p[k * h] = v[k];
            }
            __syncthreads();
        };
        radix8(1);
        radix8(8);
        // thread (token, rows c, c + 1 of the lower half of a 128-row block): the distance-64
        // butterflies of both rows, then both halves out
        for (int e = tid; e < BM * (BNW / 4); e += NT) {
            const int tl = e / (BNW / 4), q = e % (BNW / 4);
            const int c = (q / 32) * 128 + 2 * (q % 32);
            const int tok = tok0 + tl;
            if (tok < T && row0 + c < N) {  // N and row0 are multiples of 128: whole blocks
                const float* p = Ab + tl * (BNW + 1) + c;
                const float a0 = p[0], a1 = p[1], b0 = p[64], b1 = p[65];
                uint16_t* o = a.out16 + size_t(tok) * ldo + row0 + c;
                *reinterpret_cast<uint32_t*>(o) =
                    f2h((a0 + b0) * a.norm) | (f2h((a1 + b1) * a.norm) << 16);
                *reinterpret_cast<uint32_t*>(o + 64) =
                    f2h((a0 - b0) * a.norm) | (f2h((a1 - b1) * a.norm) << 16);
            }
        }
        return;
    }

    if constexpr (!PAIR) {
        // scalar LUT: row scales, then the rank-r term z U^T (split 0 only) as r / 16 more K
        // steps with both operands read straight from global memory (z rounded to binary16)
#pragma unroll
        for (int j = 0; j < RF; ++j) {
            const float sr = h2f(a.sc[0][min(wrow + 32 * j + n, N - 1)]);
#pragma unroll
            for (int i = 0; i < TF; ++i) acc[0][j][i] *= sr;
        }
        // The rank-r term's K steps of 16 are spread over the K splits (step kr / 16 in split
        // (kr / 16) % nsplit): the split planes are summed later, and no split carries it alone.
        // With r a multiple of 16 and 16-byte aligned rows a lane's 8 columns of U are one 16-byte
        // load and of z two; otherwise one element at a time.
        const bool vec = a.r % 16 == 0 && (reinterpret_cast<uintptr_t>(a.U) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(a.z) & 15) == 0;
        if (a.r > 0) {
            for (int kr = 16 * int(blockIdx.z); kr < a.r; kr += 16 * nsplit) {
                const int k0 = kr + 8 * kh;  // this lane's 8 columns of the step
                u32x4 Bu[RF];
#pragma unroll
                for (int j = 0; j < RF; ++j) {
                    const uint16_t* up = a.U + size_t(min(wrow + 32 * j + n, N - 1)) * a.r;
                    if (vec) {
                        Bu[j] = *reinterpret_cast<const u32x4*>(up + k0);
                    } else {
                        uint32_t h[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t u0 = k0 + 2 * q < a.r ? up[k0 + 2 * q] : 0u;
                            const uint32_t u1 = k0 + 2 * q + 1 < a.r ? up[k0 + 2 * q + 1] : 0u;
                            h[q] = u0 | (u1 << 16);
                        }
                        Bu[j] = u32x4{h[0], h[1], h[2], h[3]};
                    }
                }
#pragma unroll
                for (int i = 0; i < TF; ++i) {
                    // rows past T repeat row T - 1: their products are never stored
                    const int tok = tok0 + 32 * i + n;
                    const float* zp = a.z + size_t(min(tok, T - 1)) * a.r;
                    uint32_t h[4];
                    if (vec) {
                        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zp + k0);
                        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zp + k0 + 4);
                        h[0] = f2h(z0[0]) | (f2h(z0[1]) << 16);
                        h[1] = f2h(z0[2]) | (f2h(z0[3]) << 16);
                        h[2] = f2h(z1[0]) | (f2h(z1[1]) << 16);
                        h[3] = f2h(z1[2]) | (f2h(z1[3]) << 16);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float z0 = k0 + 2 * q < a.r ? zp[k0 + 2 * q] : 0.f;
                            const float z1 = k0 + 2 * q + 1 < a.r ? zp[k0 + 2 * q + 1] : 0.f;
                            h[q] = f2h(z0) | (f2h(z1) << 16);
                        }
                    }
                    const u32x4 Az = u32x4{h[0], h[1], h[2], h[3]};
#pragma unroll
                    for (int j = 0; j < RF; ++j) acc[0][j][i] = mfma32x32x16(Az, Bu[j], acc[0][j][i]);
                }
            }
        }
    }

    // whole token tiles store without a check per element
    const bool full = tok0 + BM <= T;
    // K-split planes: this split's plane ([T][N], or [T][2][N] for g and u)
    float* const plane = a.out32 + size_t(blockIdx.z) * size_t(T) * size_t(EPI == kEgPart2 ? 2 * N : N);
#pragma unroll
    for (int j = 0; j < RF; ++j) {
        const int row = wrow + 32 * j + n;
        if (wrow + 32 * j >= N) continue;  // whole 32-row operands (N is a multiple of 32)
        float s0 = 1.f, s1 = 1.f;
        bool neg = false;
        if constexpr (EPI == kEgGateUp32) {
            s0 = h2f(a.sc[0][row]);
            s1 = h2f(a.sc[1][row]);
            neg = a.sign && a.sign[row] < 0;
        } else if constexpr (EPI == kEgScale16) {
            s0 = h2f(a.sc[0][row]);
        } else if constexpr (EPI == kEgLUT || EPI == kEgLUTPlane) {
            // scaled above
        } else {
            // planes carry a scale (1 for plain partial sums): a product on the accumulators
            // here keeps them in place through the K loop, where plain stores had the register
            // allocator move them between register files on every K step
            s0 = s1 = a.norm;
        }
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int tok = tok0 + 32 * i + 8 * (q >> 2) + 4 * kh + (q & 3);
                if (!full && tok >= T) continue;
                const float v0 = acc[0][j][i][q];
                if constexpr (EPI == kEgGateUp32) {
                    const float g = v0 * s0, u = acc[NMAT - 1][j][i][q] * s1;
                    const float act = silu(g) * u;
                    a.out32[size_t(tok) * ldo + row] = neg ? -act : act;
                } else if constexpr (EPI == kEgScale16) {
                    a.out16[size_t(tok) * ldo + row] = (uint16_t)f2h(v0 * s0);
                } else if constexpr (EPI == kEgLUT) {
                    a.out16[size_t(tok) * ldo + row] = (uint16_t)f2h(v0);
                } else if constexpr (EPI == kEgPart2) {
                    // split z of a K-split gate/up product: unscaled g and u planes
                    float* o = plane + uint32_t(tok * 2 * N + row);
                    o[0] = v0 * s0;
                    o[N] = acc[NMAT - 1][j][i][q] * s1;
                } else {  // split z of a K-split product writes its own [T][N] plane
                    plane[uint32_t(tok * N + row)] = v0 * s0;
                }
            }
    }
}

// K tiles of codes in flight beyond the next one: at 64-token tiles a K tile's products take
// well under the memory latency, so the codes are requested four tiles ahead
constexpr int kCQ = 4;

template <int NW, int BM, int RW, int NMAT, int EPI, int DEC = kDecVQ3>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
    constexpr int BNW = NW * RW;
    const dim3 grid((a.N + BNW - 1) / BNW, (a.T + BM - 1) / BM, a.ksplit > 1 ? a.ksplit : 1);
    hipLaunchKernelGGL((k_vq3mm<NW, BM, RW, NMAT, DEC, EPI, kCQ>), grid, dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

// Tile shapes: waves, tokens and rows per wave of the gate/up product (two matrices) and of the
// down product (one matrix).  One wave per SIMD: the accumulators live in the AGPRs.  Prefill
// (T >= kWideT) runs the VQ3 kinds with two waves per SIMD (kWideNW per workgroup, 256 registers
// each): with one wave the decode and the matrix-core steps of a SIMD mostly take turns, with two
// one wave's decode runs beside the other's products.
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
// 128-token tiles, or 64 when T <= 64 (fewer padded rows at the fixed 64-row prefill chunk)
constexpr int kGuNW = VQ3MM_GU_NW, kGuBM = 128, kGuRW = VQ3MM_GU_RW;
constexpr int kDnNW = VQ3MM_DN_NW, kDnBM = 128, kDnRW = VQ3MM_DN_RW;
constexpr int kSmallBM = 64;
#ifndef VQ3MM_WIDE_DN_RW
#define VQ3MM_WIDE_DN_RW 64
#endif
constexpr int kWideT = 256, kWideNW = 8, kWideGuRW = 32, kWideDnRW = VQ3MM_WIDE_DN_RW;

bool vq3_kind(int kind) {
    return kind == kGemmVQ3GateUp || kind == kGemmVQ3GateUpRot || kind == kGemmVQ3GateUpSplit ||
           kind == kGemmVQ3Down || kind == kGemmVQ3DownSplit;
}
bool gateup_kind(int kind) {
    return kind == kGemmVQ3GateUp || kind == kGemmVQ3GateUpRot || kind == kGemmVQ3GateUpSplit;
}

}  // namespace

Vq3Tile vq3mm_tile(int kind, int T) {
    if (T <= kSmallBM)
        return Vq3Tile{kSmallBM, gateup_kind(kind) ? kGuNW * kGuRW : kDnNW * kDnRW};
    if (T >= kWideT && vq3_kind(kind))
        return Vq3Tile{kGuBM, gateup_kind(kind) ? kWideNW * kWideGuRW : kWideNW * kWideDnRW};
    return gateup_kind(kind) ? Vq3Tile{kGuBM, kGuNW * kGuRW} : Vq3Tile{kDnBM, kDnNW * kDnRW};
}

// DV: the decoder of the VQ kinds (VQ3, or 2x16 for a 2x16 plan)
template <int BMG, int BMD, int DV>
hipError_t launch_vq3mm_bm(const GemmArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.K % kXK || a.N <= 0 || a.N % 32) return hipErrorInvalidValue;
    if (a.ksplit > 1 && (a.K / kXK) < a.ksplit) return hipErrorInvalidValue;
    switch (a.kind) {
        case kGemmVQ3GateUp:
            return launch_t<kGuNW, BMG, kGuRW, 2, kEgGateUp32, DV>(a, st);
        case kGemmVQ3GateUpRot:  // whole 128-row rotation blocks
            if (a.N % 128) return hipErrorInvalidValue;
            return launch_t<kGuNW, BMG, kGuRW, 2, kEgGateUpRot, DV>(a, st);
        case kGemmVQ3GateUpSplit:  // the leftover rows of a larger product: 64-token tiles
            return a.bm64 ? launch_t<kGuNW, kSmallBM, kGuRW, 2, kEgPart2, DV>(a, st)
                          : launch_t<kGuNW, BMG, kGuRW, 2, kEgPart2, DV>(a, st);
        case kGemmVQ3Down:
            return launch_t<kDnNW, BMD, kDnRW, 1, kEgScale16, DV>(a, st);
        case kGemmVQ3DownSplit:
            return launch_t<kDnNW, BMD, kDnRW, 1, kEgPlain32, DV>(a, st);
        case kGemmLUT2:  // scalar LUT + rank-r term: binary16 y, or scaled FP32 planes per K split
            return a.ksplit > 1 ? launch_t<kDnNW, BMD, kDnRW, 1, kEgLUTPlane, kDecLUT2>(a, st)
                                : launch_t<kDnNW, BMD, kDnRW, 1, kEgLUT, kDecLUT2>(a, st);
        case kGemmLUT4:
            return a.ksplit > 1 ? launch_t<kDnNW, BMD, kDnRW, 1, kEgLUTPlane, kDecLUT4>(a, st)
                                : launch_t<kDnNW, BMD, kDnRW, 1, kEgLUT, kDecLUT4>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int DV>
hipError_t launch_vq3mm_wide(const GemmArgs& a, hipStream_t st) {
    if (a.K % kXK || a.N <= 0 || a.N % 32) return hipErrorInvalidValue;
    if (a.ksplit > 1 && (a.K / kXK) < a.ksplit) return hipErrorInvalidValue;
    switch (a.kind) {
        case kGemmVQ3GateUp:
            return launch_t<kWideNW, kGuBM, kWideGuRW, 2, kEgGateUp32, DV>(a, st);
        case kGemmVQ3GateUpRot:
            if (a.N % 128) return hipErrorInvalidValue;
            return launch_t<kWideNW, kGuBM, kWideGuRW, 2, kEgGateUpRot, DV>(a, st);
        case kGemmVQ3GateUpSplit:
            return a.bm64 ? launch_t<kWideNW, kSmallBM, kWideGuRW, 2, kEgPart2, DV>(a, st)
                          : launch_t<kWideNW, kGuBM, kWideGuRW, 2, kEgPart2, DV>(a, st);
        case kGemmVQ3Down:
            return launch_t<kWideNW, kDnBM, kWideDnRW, 1, kEgScale16, DV>(a, st);
        case kGemmVQ3DownSplit:
            return launch_t<kWideNW, kDnBM, kWideDnRW, 1, kEgPlain32, DV>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_vq3mm(const GemmArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    if (a.vq2 && !vq3_kind(a.kind)) return hipErrorInvalidValue;
    if (a.T <= kSmallBM)
        return a.vq2 ? launch_vq3mm_bm<kSmallBM, kSmallBM, kDecVQ2>(a, st)
                     : launch_vq3mm_bm<kSmallBM, kSmallBM, kDecVQ3>(a, st);
    if (a.T >= kWideT && vq3_kind(a.kind))
        return a.vq2 ? launch_vq3mm_wide<kDecVQ2>(a, st) : launch_vq3mm_wide<kDecVQ3>(a, st);
    return a.vq2 ? launch_vq3mm_bm<kGuBM, kDnBM, kDecVQ2>(a, st) : launch_vq3mm_bm<kGuBM, kDnBM, kDecVQ3>(a, st);
}

}  // namespace vqmlp
