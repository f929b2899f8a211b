// vq3mm.hip -- matrix-core product with the VQ3 weights decoded in registers, for T > 64 rows
// (gfx950).
//
//   D[t][n] = sum_k X[t][k] W[n][k],   X binary16 [T][K] (rotated activations), W packed VQ3.
//
// Model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP, token-mixer
// rotations, distilled weights": a six-bit code selects the pair (W[2p][j], W[2p+1][j]) from 64
// two-component binary16 centroids shared by 8 rows; row scales are applied in the epilogue.
//
// Work split.  A workgroup of NW waves (one per SIMD) owns BM tokens x NW*RW rows (of each of
// NMAT matrices that share X).  Each wave owns RW rows and all BM tokens, so no weight is used by
// two waves and the decoded weights never pass through LDS: a wave turns its own codes straight
// into the B operands of v_mfma_f32_16x16x32_f16.  Only the activation tile is staged through
// LDS, where all waves read it.
//
// Decoding.  The centroids of the two 8-row groups of a 16-row operand sit in one LDS table,
// replicated over the 32 bank columns: column b holds the first group's 64 centroids for
// b % 16 < 8 and the second group's otherwise, matching the row (lane % 16) of the lanes that
// read column lane % 32.  A lookup is one 4-byte LDS read at (code, own column), free of bank
// conflicts whatever the codes.  A centroid holds both rows of a pair, so lane n fetches the
// centroids of its pair for four of the operand's eight columns, keeps its own row's halves and
// trades the other halves with lane n ^ 1 (one DPP quad permute).  The tables are written once
// per workgroup: the codebooks are shared by all K.
//
// Column order.  Within a 64-column K tile, operand slot (ks, kg, i) -- K step ks (of 2), lane
// group kg = lane / 16, element i (of 8) -- holds column 16 (i / 2) + 4 kg + 2 ks + (i % 2).  With
// this order the codes a lane needs for one K tile are 48 contiguous bits of its pair's 96-bit
// lane record in the packed tile.  The activations are staged into LDS in the same order, so an
// A operand is still one 16-byte LDS read.
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

template <int NW, int BM, int RW, int NMAT, int EPI>
__global__ void __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_vq3mm(GemmArgs a) {
    constexpr int NT = NW * 64;
    constexpr int RF = RW / 16;       // 16-row operands per wave per matrix
    constexpr int TF = BM / 16;       // 16-token operands
    constexpr int BNW = NW * RW;      // rows per workgroup
    constexpr int NTAB = NMAT * RF;   // centroid tables per wave (one per 16-row operand)
    constexpr int XCH = BM * 8 / NT;  // 16-byte activation chunks per thread per K tile
    static_assert(RW % 32 == 0 && XCH >= 1 && (BM * 8) % NT == 0, "shape");
    constexpr int kTabBytes = 64 * 32 * 4;        // 64 centroids x 32 bank columns
    constexpr int kOffX = NW * NTAB * kTabBytes;  // activation tiles after the tables
    constexpr int kXBuf = BM * kXK * 2;           // one activation tile
    constexpr int kMain = kOffX + 2 * kXBuf;
    constexpr int kEpBytes = EPI == kEgGateUpRot ? BM * (BNW + 1) * 4 : 0;
    constexpr int kLds = kMain > kEpBytes ? kMain : kEpBytes;
    static_assert(kLds <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];

    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int n = l & 15, kg = l >> 4, c0 = n & 1, pr = n >> 1;
    const int N = a.N, K = a.K, T = a.T, KT = K / kXK;
    const int row0 = blockIdx.x * BNW, tok0 = blockIdx.y * BM;
    const int wrow = row0 + w * RW;  // first row of this wave
    const int ldo = a.ldo > 0 ? a.ldo : N;
    const int mt_last = N / 32 - 1;

    // ---- centroid tables.  Table (m, j) serves operand j of matrix m (rows wrow + 16 j ..,
    // two 8-row groups): word (e, b) -- centroid e, bank column b -- holds centroid e of the
    // first group for b % 16 < 8 and of the second group otherwise.  Lane l reads column l % 32
    // only, which holds its own row's group, so a lookup never meets a bank conflict.
    {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const uint32_t* cb = (NMAT > 1 && m) ? a.cb[1] : a.cb[0];
#pragma unroll
            for (int j = 0; j < RF; ++j) {
                unsigned char* tb = lds + (w * NTAB + m * RF + j) * kTabBytes;
                const int g0 = wrow / 8 + 2 * j;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int idx = l + 64 * k, e = idx >> 3, bq = idx & 7;  // 4 columns per store
                    const int grp = min(g0 + ((bq >> 1) & 1), N / 8 - 1);
                    const uint32_t v = cb[size_t(grp) * 64 + e];
                    *reinterpret_cast<u32x4*>(tb + e * 128 + bq * 16) = u32x4{v, v, v, v};
                }
            }
        }
    }
    const uint32_t tab_lane = uint32_t(w * NTAB * kTabBytes) + uint32_t(l & 31) * 4u;

    // ---- this lane's codes.  Lane (row n of an operand: pair pr, component c0) looks up the
    // centroids of its own pair for operand columns 4 c0 .. 4 c0 + 3, i.e. record slots 2 c0 and
    // 2 c0 + 1 of lane record (kg, pair) -- record bits 48 c0 .. 48 c0 + 47, inside the two words
    // starting at word c0.
    uint32_t voff[RF];
#pragma unroll
    for (int j = 0; j < RF; ++j) {
        const int mt = min(wrow / 32 + j / 2, mt_last);
        const int pp = 8 * (j & 1) + pr;
        voff[j] = uint32_t(mt) * uint32_t(KT) * kTileBytes + 12u * uint32_t((kg << 4) | pp) +
                  4u * uint32_t(c0);
    }
    const uint32_t sh16 = 16u * uint32_t(c0);
    // v_perm selectors: this lane's component and the partner's
    const uint32_t sel_own = c0 ? 0x07060302u : 0x05040100u;
    const uint32_t sel_oth = c0 ? 0x05040100u : 0x07060302u;

    // ---- activation tiles in LDS: row r (token), 16-byte chunk q (operand positions 8q ..
    // 8q + 7, i.e. K step q / 4 and lane group q % 4) stored at chunk q ^ (r % 8), so that the
    // eight rows read together hit eight different chunks.
    const uint32_t aoff0 = kOffX + uint32_t(n) * 128u + (uint32_t(kg ^ (n & 7)) << 4);
    const uint32_t aoff1 = kOffX + uint32_t(n) * 128u + (uint32_t((4 + kg) ^ (n & 7)) << 4);
    // staging: this thread's chunk x holds token row c / 8, columns 8 (c % 8) .. + 7; its four
    // words go to operand chunks 2 (u % 2) + {0, 4, 1, 5}, word u / 2 of each
    // (chunk x is NT / 8 rows below chunk 0, with the same row % 8: a constant offset)
    uint32_t xw[4];
    uint32_t xoff[XCH];  // global byte offset of the chunk in K tile 0
    static_assert((NT / 8) % 8 == 0, "chunks of one thread share the row swizzle");
    {
        const int tt = tid >> 3, u = tid & 7;
        constexpr int qd[4] = {0, 4, 1, 5};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int q = 2 * (u & 1) + qd[d];
            xw[d] = kOffX + uint32_t(tt) * 128u + (uint32_t(q ^ (tt & 7)) << 4) + 4u * uint32_t(u >> 1);
        }
    }
#pragma unroll
    for (int x = 0; x < XCH; ++x) {
        const int c = tid + x * NT;
        const int tt = c >> 3, u = c & 7;
        // rows past T repeat row T - 1: their products are never stored
        const int tok = min(tok0 + tt, T - 1);
        xoff[x] = (uint32_t(tok) * uint32_t(K) + 8u * uint32_t(u)) * 2u;
    }

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

    u32x4 xr[XCH];          // activation chunks of the next K tile
    u32x2 cw[NMAT][RF];     // code windows of the next K tile
    u32x4 Bf[2][NMAT][RF];  // B operands [ks][m][j]

    auto load_x = [&](int kt) {
#pragma unroll
        for (int x = 0; x < XCH; ++x)
            xr[x] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, int(xoff[x]), kt * kXK * 2, 0));
    };
    auto load_codes = [&](int kt) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j)
                cw[m][j] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs_code[m], int(voff[j]),
                                                                kt * kTileBytes, 0));
    };
    auto stage = [&](uint32_t bufoff) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            unsigned char* base = lds + (xw[d] + bufoff);
#pragma unroll
            for (int x = 0; x < XCH; ++x)
                *reinterpret_cast<uint32_t*>(base + x * (NT / 8) * 128) = xr[x][d];
        }
    };

    // the lane's 48-bit code field of every record of one K tile, as low word and high half-word
    uint32_t flo[NMAT][RF], fhi[NMAT][RF];
    auto extract = [&]() {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j) {
                const u32x2 v = cw[m][j];
                flo[m][j] = __builtin_amdgcn_alignbit(v[1], v[0], sh16);
                fhi[m][j] = v[1] >> sh16;
            }
    };

    // Decoding B operand (ks, m, j) from the current code fields, in two phases: the four table
    // reads (centroids of columns 4 c0 .. 4 c0 + 3 of the lane's pair), then the exchange with
    // lane n ^ 1 that gives each lane its own component at all eight columns.
    constexpr int NB = NMAT * RF;  // B operands per K step
    uint32_t ev[2][4];             // table reads of two operands in flight
    auto dec_read = [&](int ks, int b) {
        const int m = b / RF, j = b % RF;
        const uint32_t lo = flo[m][j], hi = fhi[m][j];
        // code k of the operand at field bit 24 (k / 2) + 12 ks + 6 (k % 2), moved to bits 12:7
        uint32_t x0, x1, x2, x3;
        if (ks == 0) {
            x0 = lo << 7;
            x1 = lo << 1;
            x2 = lo >> 17;
            x3 = __builtin_amdgcn_alignbit(hi, lo, 23);
        } else {
            x0 = lo >> 5;
            x1 = lo >> 11;
            x2 = hi << 3;
            x3 = hi >> 3;
        }
        const unsigned char* tb = lds + b * kTabBytes;
        ev[b & 1][0] = *reinterpret_cast<const uint32_t*>(tb + and_or(x0, 0x1F80u, tab_lane));
        ev[b & 1][1] = *reinterpret_cast<const uint32_t*>(tb + and_or(x1, 0x1F80u, tab_lane));
        ev[b & 1][2] = *reinterpret_cast<const uint32_t*>(tb + and_or(x2, 0x1F80u, tab_lane));
        ev[b & 1][3] = *reinterpret_cast<const uint32_t*>(tb + and_or(x3, 0x1F80u, tab_lane));
    };
    auto dec_place = [&](int ks, int b) {
        const int m = b / RF, j = b % RF;
        const uint32_t e0 = ev[b & 1][0], e1 = ev[b & 1][1], e2 = ev[b & 1][2], e3 = ev[b & 1][3];
        const uint32_t y0 = __builtin_amdgcn_perm(e1, e0, sel_own);
        const uint32_t y1 = __builtin_amdgcn_perm(e3, e2, sel_own);
        const uint32_t r0 = from_xor1(__builtin_amdgcn_perm(e1, e0, sel_oth));
        const uint32_t r1 = from_xor1(__builtin_amdgcn_perm(e3, e2, sel_oth));
        Bf[ks][m][j] = c0 ? u32x4{r0, r1, y0, y1} : u32x4{y0, y1, r0, r1};
    };

    f32x4 acc[NMAT][RF][TF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < RF; ++j)
#pragma unroll
            for (int i = 0; i < TF; ++i) acc[m][j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto readA = [&](uint32_t bufoff, int ks, int i) {
        return *reinterpret_cast<const u32x4*>(lds + (ks ? aoff1 : aoff0) + bufoff + i * 2048);
    };
    auto mma_unit = [&](int ks, int i, const u32x4& A) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int j = 0; j < RF; ++j) acc[m][j][i] = mfma16x16x32(A, Bf[ks][m][j], acc[m][j][i]);
    };

    // this workgroup's K tiles: split blockIdx.z of a.ksplit equal ranges
    const int nsplit = a.ksplit > 1 ? a.ksplit : 1;
    const int kb = int(blockIdx.z) * KT / nsplit, nk = (int(blockIdx.z) + 1) * KT / nsplit - kb;
    auto tile = [&](int t) { return kb + min(t, nk - 1); };  // loads past the end repeat the last

    // Prologue: tables, tile 0's activations in buffer 0, its K step 0 operands decoded; the
    // codes and activations of tile 1 requested.
    load_codes(tile(0));
    load_x(tile(0));
    __syncthreads();  // tables
    extract();
    load_codes(tile(1));
    stage(0);
    load_x(tile(1));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        dec_read(0, b);
        dec_place(0, b);
    }
    __syncthreads();

    // One K step per iteration, hand-interleaved.  The products of tile t run in 2 TF units (one
    // A operand, NB matrix-core steps each): the first TF (K step 0) beside the decoding of the
    // tile's K step 1 operands, the last TF (K step 1) beside the decoding of tile t + 1's K step 0
    // operands, each into the registers its products have just released.  Mid-step the code
    // fields of tile t + 1 are taken (once the last read of tile t's has gone out) and tile t + 2's
    // codes requested; at the end tile t + 1's
    // activations are staged and tile t + 2's requested.  A operands are read two units ahead;
    // scheduling barriers keep this order.  Every load is unconditional, so each wait counts the
    // same loads on every path.
    static_assert(TF == 2 * NB, "two product units per decoded operand");
    for (int t = 0; t < nk; ++t) {
        const uint32_t cur = uint32_t(t & 1) * kXBuf, nxt = uint32_t(kXBuf) - cur;
        u32x4 Ar[3];
        Ar[0] = readA(cur, 0, 0);
        Ar[1] = readA(cur, 0, 1);
        dec_read(1, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2 * TF; ++c) {
            const int ks = c / TF, i = c % TF;
            if (c + 2 < 2 * TF) Ar[(c + 2) % 3] = readA(cur, (c + 2) / TF, (c + 2) % TF);
            mma_unit(ks, i, Ar[c % 3]);
            if (c == TF - 2) {  // tile t's codes are read: take tile t + 1's, request t + 2's
                extract();
                load_codes(tile(t + 2));
            }
            if (c % 2 == 0) {
                // operand b of the K step being decoded: (tile t, ks 1) in the first half,
                // (tile t + 1, ks 0) in the second
                const int dk = ks == 0 ? 1 : 0, b = i / 2;
                if (b + 1 < NB) dec_read(dk, b + 1);
                else if (ks == 0) dec_read(0, 0);  // first operand of the second half
            } else {
                const int dk = ks == 0 ? 1 : 0, b = i / 2;
                dec_place(dk, b);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        stage(nxt);  // activations of tile t + 1
        load_x(tile(t + 2));
        __syncthreads();
    }
    if constexpr (EPI == kEgGateUpRot) __syncthreads();  // the epilogue reuses the LDS

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

    // whole token tiles store without a check per element
    const bool full = tok0 + BM <= T;
    // K-split planes: this split's plane ([T][N], or [T][2][N] for g and u)
    float* const plane = a.out32 + size_t(blockIdx.z) * size_t(T) * size_t(EPI == kEgPart2 ? 2 * N : N);
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
        } else {
            // planes carry a scale (1 for plain partial sums): a product on the accumulators
            // here keeps them in place through the K loop, where plain stores had the register
            // allocator move them between register files on every K step
            s0 = s1 = a.norm;
        }
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int tok = tok0 + 16 * i + 4 * kg + q;
                if (!full && tok >= T) continue;
                const float v0 = acc[0][j][i][q];
                if constexpr (EPI == kEgGateUp32) {
                    const float g = v0 * s0, u = acc[NMAT - 1][j][i][q] * s1;
                    const float act = g / (1.f + expf(-g)) * u;
                    a.out32[size_t(tok) * ldo + row] = neg ? -act : act;
                } else if constexpr (EPI == kEgScale16) {
                    a.out16[size_t(tok) * ldo + row] = (uint16_t)f2h(v0 * s0);
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
