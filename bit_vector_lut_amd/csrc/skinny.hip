// skinny.hip -- bandwidth-bound VQ3 projection for T <= 8 rows (gfx950).
//
// Weight format (model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit
// MLP, token-mixer rotations, distilled weights"): six-bit codes select one of 64 two-component
// binary16 centroids shared by 8 output rows; each code gives (W[2p][j], W[2p+1][j]).
//
// Product.  v_mfma_f32_16x16x32_f16 with
//   A (16 x 32): row i = row pair 16*mt + i; column 2*jj + c = component c of the centroid that
//                code[pair][16*step + jj] selects, i.e. the 32-bit table entry as it is;
//   B (32 x 16): B[2*jj + c][2*t + c'] = x~[t][16*step + jj] if c == c' else 0;
// so D[i][2t + c'] is row 2*(16*mt + i) + c' of W x~ for token t.  Eight tokens times two
// components fill the 16 columns and the decoded pairs need no repacking.
//
// Lookups.  Each code is looked up in LDS: entry c of the table lane l uses is dword 32*c + l%32
// of a 2048-dword table, so each 32-lane half of a lookup touches 32 different banks.  The
// address is two VALU ops (align the code to bit 7, and-or the lane base).
//
// Work.  A workgroup of 16 waves (4 per SIMD: the VALU issues fast only with several waves per
// SIMD) owns one work item at a time: two 16-pair row tiles (gate and up of the same rows, or
// two neighbouring tiles of down) that share the activation operand, times one K slice.  Wave w
// owns tiles [w*TPW, (w+1)*TPW) of the slice and keeps its activation operand in registers.
// Code words are prefetched D tiles ahead through a register ring that runs on across work
// items; every load is consumed within the iteration that issues it, so the in-order memory
// counter never forces a drain of the prefetch.  Tiles past K multiply a zero operand (their
// code loads are clamped to a valid tile), so the tile loop has no control flow.
#include "device.h"
#include "internal.h"

namespace vqmlp {

constexpr int kTabDwords = 64 * 32;
constexpr int kWaves = kSkinnyWaves;

template <int TPW, int D, int EPI>
__global__ void __launch_bounds__(kWaves * 64, 1) k_stream(SkinnyArgs a) {
    static_assert(TPW % D == 0, "ring depth must divide the tiles per wave");
    __shared__ uint32_t tab[2][2][kTabDwords];
    __shared__ f32x4 red[kWaves][2][64];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int K = a.mat[0].K, N = a.mat[0].N;
    const int KT = K / kTileCols, MT = N / kTileRows;
    // a work item: slice sl and row-tile pair q (gate/up: both matrices at tile q; down: tiles
    // 2q and 2q+1 of the one matrix)
    const int NQ = EPI == kEpiGateUp ? MT : (MT + 1) / 2;
    const int items = a.slices * NQ;
    const int G = gridDim.x;
    int first, last, step;
    if (a.contig) {
        first = int((long long)blockIdx.x * items / G);
        last = int((long long)(blockIdx.x + 1) * items / G);
        step = 1;
    } else {
        first = blockIdx.x;
        last = items;
        step = G;
    }
    if (first >= last) return;
    auto tile_of = [&](int q, int m) -> int {
        if (EPI == kEpiGateUp) return q;
        const int t = 2 * q + m;
        return t < MT ? t : MT - 1;
    };

    // operand selectors: lane l holds column n = l%16 = 2*tok + cp of B
    const int n = l & 15, tok = n >> 1, cp = n & 1;
    const uint32_t sel_e = cp ? 0x05040C0Cu : 0x0C0C0504u;  // (x_lo, 0) or (0, x_lo)
    const uint32_t sel_o = cp ? 0x07060C0Cu : 0x0C0C0706u;  // (x_hi, 0) or (0, x_hi)
    const uint32_t lane4 = uint32_t(l & 31) << 2;

    // codebook word this thread turns into 2 x 4 table dwords (threads 0..511)
    const int cb_m = (tid >> 8) & 1, cb_g = (tid >> 6) & 3, cb_c = tid & 63;
    const bool cb_thread = tid < 512;
    const uint32_t* cb_base = cb_m ? a.mat[1].cb : a.mat[0].cb;  // uniform per wave
    auto cb_load = [&](int idx) -> uint32_t {
        const int mt = tile_of(idx % NQ, cb_m);
        return cb_base[size_t(mt * 4 + cb_g) * 64 + cb_c];
    };
    auto write_tables = [&](int buf, uint32_t v) {
        if (cb_thread) {
            const u32x4 q = u32x4{v, v, v, v};
            *reinterpret_cast<u32x4*>(&tab[buf][cb_m][cb_c * 32 + 4 * cb_g]) = q;
            *reinterpret_cast<u32x4*>(&tab[buf][cb_m][cb_c * 32 + 4 * (cb_g + 4)]) = q;
        }
    };
    // tiles of item idx that exist for this wave; tiles past K are clamped to the last one
    auto item_tiles = [&](int idx, int& kt0, int& last_kt, int& ntile) {
        const int sl = idx / NQ;
        kt0 = (sl * kWaves + w) * TPW;
        ntile = KT - kt0;
        ntile = ntile < TPW ? (ntile > 0 ? ntile : 0) : TPW;
        last_kt = kt0 + (ntile > 0 ? ntile : 1) - 1;
        last_kt = last_kt < KT ? last_kt : KT - 1;
    };
    auto tile_word = [&](int m, int idx, int kt) -> const uint32_t* {
        const int mt = tile_of(idx % NQ, m);
        return reinterpret_cast<const uint32_t*>(a.mat[m].codes +
                                                 (size_t(mt) * KT + kt) * kTileBytes) + 3 * l;
    };

    uint32_t ring[D][2][3];
    int idx = first;
    if (cb_thread) write_tables(0, cb_load(idx));
    int kt0, last_kt, ntile;
    item_tiles(idx, kt0, last_kt, ntile);
#pragma unroll
    for (int t = 0; t < D; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int kt = kt0 + t < last_kt ? kt0 + t : last_kt;
            const uint32_t* p = tile_word(m, idx, kt);
            ring[t][m][0] = p[0];
            ring[t][m][1] = p[1];
            ring[t][m][2] = p[2];
        }

    int cur_slice = -1;
    uint32_t B[TPW * 4][2];
    for (int j = 0;; ++j) {
        const int buf = j & 1;
        const int nidx = idx + step < last ? idx + step : -1;
        // loads for the next item are issued unconditionally (the last item reloads itself)
        const int pidx = nidx >= 0 ? nidx : idx;
        const uint32_t cbv_next = cb_thread ? cb_load(pidx) : 0u;
        const int sl = idx / NQ, q = idx % NQ;
        int nkt0, nlast_kt, nntile;
        item_tiles(pidx, nkt0, nlast_kt, nntile);
        if (sl != cur_slice) {
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kt = kt0 + t < KT ? kt0 + t : KT - 1;
                    const u32x2 v = *reinterpret_cast<const u32x2*>(
                        a.bx + size_t(tok) * K + kt * kTileCols + 16 * s + 4 * (l >> 4));
                    const bool ok = t < ntile;  // tiles past K multiply a zero operand
                    B[t * 4 + s][0] = ok ? v[0] : 0u;
                    B[t * 4 + s][1] = ok ? v[1] : 0u;
                }
            cur_slice = sl;
        }
        uint32_t laneb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) laneb[m] = lane4 | uint32_t((buf * 2 + m) * kTabDwords * 4);
        const char* tbase = reinterpret_cast<const char*>(&tab[0][0][0]);

        // epilogue operands, fetched now so that waiting for them later does not drain the
        // code prefetch issued after them.  Thread e < 512 owns output (slot e/256, reg, lane).
        const int e_m = (tid >> 8) & 1, e_r = (tid >> 6) & 3, e_l = tid & 63;
        const int e_mt = tile_of(q, EPI == kEpiGateUp ? 0 : e_m);
        const int e_row = e_mt * kTileRows + 2 * (4 * (e_l >> 4) + e_r) + (e_l & 1);
        const bool e_thread = EPI == kEpiGateUp ? tid < 256 : tid < 512;
        uint32_t e_sc0 = a.mat[0].sc[e_thread ? e_row : 0];
        uint32_t e_sc1 = EPI == kEpiGateUp ? uint32_t(a.mat[1].sc[e_thread ? e_row : 0]) : 0u;
        // sign of the intermediate rotation as a float sign-bit mask (loaded unconditionally,
        // from the scales when there is no sign array, and masked; no early compare)
        const int8_t* sgn = a.sign_i ? a.sign_i : reinterpret_cast<const int8_t*>(a.mat[0].sc);
        const uint32_t sgn_mask = (EPI == kEpiGateUp && a.sign_i) ? 0x80u : 0u;
        const uint32_t e_signbit = uint32_t(uint8_t(sgn[e_thread ? e_row : 0])) & sgn_mask;
        __syncthreads();

        auto look = [&](const uint32_t (&c)[2][3], int s, u32x4 (&A)[2]) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const uint32_t d0 = c[m][0], d1 = c[m][1], d2 = c[m][2], lb = laneb[m];
#define VQ_LOOK(i, Q) A[m][i] = *reinterpret_cast<const uint32_t*>(tbase + code_addr<Q, 7>(d0, d1, d2, lb))
                if (s == 0) { VQ_LOOK(0, 0); VQ_LOOK(1, 1); VQ_LOOK(2, 2); VQ_LOOK(3, 3); }
                if (s == 1) { VQ_LOOK(0, 4); VQ_LOOK(1, 5); VQ_LOOK(2, 6); VQ_LOOK(3, 7); }
                if (s == 2) { VQ_LOOK(0, 8); VQ_LOOK(1, 9); VQ_LOOK(2, 10); VQ_LOOK(3, 11); }
                if (s == 3) { VQ_LOOK(0, 12); VQ_LOOK(1, 13); VQ_LOOK(2, 14); VQ_LOOK(3, 15); }
#undef VQ_LOOK
            }
        };
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        // A operands of consecutive steps alternate between two register sets; a ring slot is
        // refilled right after its last lookup, so the refill reuses its registers.
        u32x4 A[2][2];
        look(ring[0], 0, A[0]);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int cp0 = (4 * t + s) & 1, cp1 = cp0 ^ 1;
                if (s < 3)
                    look(ring[t % D], s + 1, A[cp1]);
                else if (t + 1 < TPW)
                    look(ring[(t + 1) % D], 0, A[cp1]);
                if (s == 2) {
                    // refill: tile t + D of this item, or tile t + D - TPW of the next one
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const uint32_t* p;
                        if (t + D < TPW) {
                            const int kt = kt0 + t + D < last_kt ? kt0 + t + D : last_kt;
                            p = tile_word(m, idx, kt);
                        } else {
                            const int kt = nkt0 + t + D - TPW < nlast_kt ? nkt0 + t + D - TPW : nlast_kt;
                            p = tile_word(m, pidx, kt);
                        }
                        ring[t % D][m][0] = p[0];
                        ring[t % D][m][1] = p[1];
                        ring[t % D][m][2] = p[2];
                    }
                    // keep the refill here: left to itself the scheduler sinks every refill to
                    // the end of the item, which exposes a full memory latency per item
                    __builtin_amdgcn_sched_barrier(0);
                }
                const uint32_t b0 = B[t * 4 + s][0], b1 = B[t * 4 + s][1];
                const u32x4 Bx = u32x4{__builtin_amdgcn_perm(b0, 0u, sel_e),
                                       __builtin_amdgcn_perm(b0, 0u, sel_o),
                                       __builtin_amdgcn_perm(b1, 0u, sel_e),
                                       __builtin_amdgcn_perm(b1, 0u, sel_o)};
                acc[0] = mfma16x16x32(A[cp0][0], Bx, acc[0]);
                acc[1] = mfma16x16x32(A[cp0][1], Bx, acc[1]);
            }
        }
        // next item's tables go to the idle buffer (its last reader finished before this
        // item's first barrier)
        write_tables(buf ^ 1, cbv_next);
        red[w][0][l] = acc[0];
        red[w][1][l] = acc[1];
        __syncthreads();
        if (e_thread) {
            const int t = (e_l & 15) >> 1;
            if (EPI == kEpiGateUp) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    g += red[ww][0][e_l][e_r];
                    u += red[ww][1][e_l][e_r];
                }
                g *= h2f(e_sc0);
                u *= h2f(e_sc1);
                const float act = g / (1.f + expf(-g)) * u;
                a.a_out[size_t(t) * N + e_row] =
                    __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, act) ^ (e_signbit << 24));
            } else {
                float v = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) v += red[ww][e_m][e_l][e_r];
                const bool valid = 2 * q + e_m < MT;
                if (EPI == kEpiDownFinal) {
                    if (valid && t < a.T) a.y[size_t(t) * N + e_row] = (uint16_t)f2h(v * h2f(e_sc0));
                } else {
                    if (valid) a.part[(size_t(sl) * kSkinnyT + t) * N + e_row] = v;
                }
            }
        }
        if (nidx < 0) break;
        idx = nidx;
        kt0 = nkt0;
        last_kt = nlast_kt;
        ntile = nntile;
    }
}

template <int TPW, int D, int EPI>
static hipError_t launch_stream_t(const SkinnyArgs& a, hipStream_t st) {
    const int MT = a.mat[0].N / kTileRows;
    const int items = a.slices * (EPI == kEpiGateUp ? MT : (MT + 1) / 2);
    // as many workgroups as keep every one at the same item count: a partial last round of
    // items would leave most of the chip idle while a few workgroups finish
    const int per = (items + 255) / 256;
    const int grid = (items + per - 1) / per;
    hipLaunchKernelGGL((k_stream<TPW, D, EPI>), dim3(grid), dim3(kWaves * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_skinny(const SkinnyArgs& in, hipStream_t st) {
    // the kernel always reads two matrix slots: a single matrix (down) fills both, its tiles
    // 2q and 2q+1 being the two row tiles of a work item
    SkinnyArgs a = in;
    if (a.nmat == 1) a.mat[1] = a.mat[0];
    for (int m = 0; m < 2; ++m)
        if (!a.mat[m].codes || !a.mat[m].cb || !a.mat[m].sc || a.mat[m].N != a.mat[0].N ||
            a.mat[m].K != a.mat[0].K)
            return hipErrorInvalidValue;
    if (!a.bx || (a.nmat == 2 && !a.a_out) || (a.nmat == 1 && a.slices == 1 && !a.y) ||
        (a.nmat == 1 && a.slices > 1 && !a.part))
        return hipErrorInvalidValue;
    const int epi = a.nmat == 2 ? kEpiGateUp : (a.slices == 1 ? kEpiDownFinal : kEpiDownPart);
#define VQ_CASE(TP, DD)                                                                  \
    if (a.tpw == TP) {                                                                   \
        if (epi == kEpiGateUp) return launch_stream_t<TP, DD, kEpiGateUp>(a, st);        \
        if (epi == kEpiDownFinal) return launch_stream_t<TP, DD, kEpiDownFinal>(a, st);  \
        return launch_stream_t<TP, DD, kEpiDownPart>(a, st);                             \
    }
    VQ_CASE(1, 1) VQ_CASE(2, 2) VQ_CASE(3, 3) VQ_CASE(4, 4) VQ_CASE(5, 5)
#undef VQ_CASE
    return hipErrorInvalidValue;
}

__global__ void __launch_bounds__(256) k_reduce_down(int T, int N, int slices, const float* part,
                                                     const uint16_t* sc, uint16_t* y) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= T * N) return;
    const int t = i / N, row = i % N;
    float sum = 0.f;
    for (int s = 0; s < slices; ++s) sum += part[(size_t(s) * kSkinnyT + t) * N + row];
    y[i] = (uint16_t)f2h(sum * h2f(sc[row]));
}

hipError_t launch_reduce_down(int T, int N, int slices, const float* part, const uint16_t* sc,
                              uint16_t* y, hipStream_t st) {
    hipLaunchKernelGGL(k_reduce_down, dim3((T * N + 255) / 256), dim3(256), 0, st, T, N, slices,
                       part, sc, y);
    return hipGetLastError();
}

}  // namespace vqmlp
