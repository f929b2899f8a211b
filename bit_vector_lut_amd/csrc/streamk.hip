// streamk.hip -- T <= 8 projections as an even split of the weight stream (gfx950).
//
// Weight format (model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit
// MLP, token-mixer rotations, distilled weights"): six-bit codes select one of 64 two-component
// binary16 centroids shared by 8 output rows; each code gives (W[2p][j], W[2p+1][j]).
//
// At T <= 8 the forward reads every weight once and does little else: its speed is the rate at
// which the chip streams the packed codes.  This kernel keeps that stream even and unbroken:
//
// Units.  A unit is one 64-column K tile of a row-tile pair (gate and up tiles q of the same 32
// rows, or down tiles 2q and 2q + 1), in q-major order; the U = NQ * KT units are cut into G
// contiguous ranges whose lengths differ by at most one, one per workgroup, and each range into
// 16 contiguous sub-ranges, one per wave.  Every wave streams its sub-range through a register
// ring (code words and activation words of kRing units ahead) with no barrier until it is done;
// a sub-range is never longer than KT, so it touches at most two row-tile pairs and the wave
// keeps two accumulator sets.
//
// Product.  v_mfma_f32_16x16x32_f16 exactly as in the per-phase kernels: A row i = row pair i of
// the tile, columns = the two components of the centroids of 16 codes (the 32-bit table entries
// as they are); B holds x~[t][.] in column 2t + c for component c, zero elsewhere.
//
// Lookups.  The tables of every row-tile pair of the workgroup's range (at most kMaxQ) sit in
// LDS for the whole launch: entry c of the table that lane l uses is dword 32 c + l % 32, so each
// 32-lane half of a lookup touches 32 different banks.
//
// Reduction.  At the end the 16 waves' partial sums of each row-tile pair are summed in LDS, in
// wave order, and written to slot q + b of the partial-sum array (slots of one q are the
// workgroups b whose ranges touch it, consecutive); a small pass sums the slots of each q in
// workgroup order and applies the epilogue, so the result does not depend on timing.
#include "device.h"
#include "internal.h"

namespace vqmlp {

namespace {
constexpr int kW = 16;                    // waves per workgroup
constexpr int kRing = 3;                  // units in flight per wave
constexpr int kMaxQ = kStreamKMaxQ;       // row-tile pairs per workgroup range
constexpr int kTabDw = 64 * 32;           // one table: 64 entries x 32 bank columns
constexpr int kSlot = 2 * 64 * 4;         // floats per partial-sum slot: 2 tiles x 64 lanes x 4
constexpr int kRsrcWord3 = 0x00020000;    // buffer resource word 3: 32-bit raw data
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// first unit of workgroup b's range
__host__ __device__ __forceinline__ int sk_start(int b, int U, int G) {
    return int((long long)b * U / G);
}
// the workgroup whose range holds unit u (U G < 2^31, checked by the launcher)
__device__ __forceinline__ int sk_owner(int u, int U, int G) {
    return int((uint32_t(u + 1) * uint32_t(G) + uint32_t(U) - 1u) / uint32_t(U)) - 1;
}
// first unit of workgroup b's range, 32-bit form of sk_start for the combine passes
__device__ __forceinline__ int sk_start32(int b, int U, int G) {
    return int(uint32_t(b) * uint32_t(U) / uint32_t(G));
}
}  // namespace

// f(std::integral_constant<int, I>) for I = B .. E - 1, in order
template <int B, int E, class F>
__device__ __forceinline__ void sk_static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        sk_static_for<B + 1, E>(f);
    }
}

template <int NMAT>
__global__ void __launch_bounds__(kW * 64, 1) k_streamk(StreamKArgs a) {
    // one LDS block with the tables at address 0: a lookup address is then the code and lane
    // bits alone (a base of 64 KB would not fit the 16-bit offset field and cost an add each)
    constexpr int kOffRed = kMaxQ * 2 * kTabDw * 4, kOffMeta = kOffRed + kW * 2 * 2 * 64 * 16;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kOffMeta + kW * 8];
    auto& tab = *reinterpret_cast<uint32_t (*)[kMaxQ][2][kTabDw]>(lds);      // 64 KB
    auto& red = *reinterpret_cast<f32x4 (*)[kW][2][2][64]>(lds + kOffRed);  // 64 KB
    auto& meta = *reinterpret_cast<int (*)[kW][2]>(lds + kOffMeta);         // wave's first, last pair
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KT = a.KT, U = a.U, MT = a.MT, G = gridDim.x, b = blockIdx.x;
    const int K = KT * kTileCols;
    const int u0 = __builtin_amdgcn_readfirstlane(sk_start(b, U, G));
    const int u1 = __builtin_amdgcn_readfirstlane(sk_start(b + 1, U, G));
    if (u0 >= u1) return;  // whole workgroup: no barrier is reached
    const int q0 = __builtin_amdgcn_readfirstlane(u0 / KT);
    const int nq = __builtin_amdgcn_readfirstlane((u1 - 1) / KT) - q0 + 1;
    auto tile_of = [&](int q, int m) -> int {
        if constexpr (NMAT == 2) return q;
        const int t = 2 * q + m;
        return t < MT ? t : MT - 1;
    };

    // ---- this wave's units [wu0, wu0 + nw): na of them in its first row-tile pair
    // (integer division runs on the vector unit: the results are made scalar again by hand, else
    // every buffer load with a scalar offset from them becomes a waterfall loop)
    const int n = u1 - u0;
    const int wu0 = __builtin_amdgcn_readfirstlane(u0 + (w * n) / kW);
    const int nw = __builtin_amdgcn_readfirstlane(u0 + ((w + 1) * n) / kW - wu0);
    const int qa = __builtin_amdgcn_readfirstlane(wu0 / KT);
    const int na = min(nw, (qa + 1) * KT - wu0);

    // operand selectors: lane l holds column n = l % 16 = 2 tok + cp of B
    const int n16 = l & 15, tok = n16 >> 1, cp = n16 & 1;
    const uint32_t sel_e = cp ? 0x05040C0Cu : 0x0C0C0504u;  // (x_lo, 0) or (0, x_lo)
    const uint32_t sel_o = cp ? 0x07060C0Cu : 0x0C0C0706u;  // (x_hi, 0) or (0, x_hi)
    const uint32_t lane4 = uint32_t(l & 31) << 2;
    const char* tbase = reinterpret_cast<const char*>(&tab[0][0][0]);
    // Loads go through buffer resources: the lane's offset is fixed, the unit's offset rides in
    // the scalar offset, so no per-lane address is kept or computed per load.
    __amdgpu_buffer_rsrc_t rs_code[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
        rs_code[m] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.mat[m].codes), 0, int(uint32_t(MT) * uint32_t(KT) * kTileBytes),
            kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.bx), 0, int(uint32_t(kSkinnyT) * uint32_t(K) * 2u), kRsrcWord3);
    const int voff_c = 12 * l;                              // the lane's 12 code bytes
    const int voff_b = ((l >> 4) * 8 + tok) * 32;           // the lane's 32 activation bytes

    // table words of this thread (loaded first: they are small and the ring waits on nothing)
    constexpr int kTabPer = (kMaxQ * 512 + kW * 64 - 1) / (kW * 64);
    uint32_t tv[kTabPer];
#pragma unroll
    for (int k = 0; k < kTabPer; ++k) {
        const int i = tid + k * kW * 64;
        const int c = i & 63, g = (i >> 6) & 3, m = (i >> 8) & 1, r = i >> 9;
        // (a select of the two pointers: indexing the argument array by a lane's m would load it)
        const uint32_t* cbm = m ? a.mat[1].cb : a.mat[0].cb;
        tv[k] = i < nq * 512 ? cbm[size_t(tile_of(q0 + r, m) * 4 + g) * 64 + c] : 0u;
    }

    // ring: code words of both tiles and the activation words of kRing units
    uint32_t rc[kRing][2][3];
    u32x4 rb[kRing][2];
    // prefetch cursor (unit index within the wave's run, clamped to the last unit)
    int pu = 0, pq = qa, pkt = wu0 - qa * KT;
    auto load_unit = [&](int j) {
        // (the cursor is uniform, but the compiler may keep it in vector registers: its
        // scalar offsets are read back from lane 0)
        const int sb = __builtin_amdgcn_readfirstlane(pkt * (kTileCols * kSkinnyT * 2));
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int sc = __builtin_amdgcn_readfirstlane((tile_of(pq, m) * KT + pkt) * kTileBytes);
            const u32x3 v = __builtin_bit_cast(
                u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs_code[m], voff_c, sc, 0));
            rc[j][m][0] = v[0];
            rc[j][m][1] = v[1];
            rc[j][m][2] = v[2];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
            rb[j][h] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_b, voff_b + 16 * h, sb, 0));
        // advance without branches: a branch here lets the compiler turn the repeated last
        // unit into register copies, which wait for the loads they copy
        const int adv = pu + 1 < nw ? 1 : 0;
        pu += adv;
        pkt += adv;
        const int wrap = pkt == KT ? 1 : 0;
        pkt -= wrap * KT;
        pq += wrap;
    };
    // in slot order (the loop head's wait for slot 0 counts on it being the oldest), before the
    // tables: the first code words are on their way while the tables load.  A wave with no
    // units loads a valid unit too (its run starts inside the range) and never reads it.
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
        load_unit(j);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- tables of the range's row-tile pairs (thread i: pair r, matrix m, group g, entry c),
    // stored once the loads (issued before the ring's) are in
#pragma unroll
    for (int k = 0; k < kTabPer; ++k) {
        const int i = tid + k * kW * 64;
        if (i < nq * 512) {
            const int c = i & 63, g = (i >> 6) & 3, m = (i >> 8) & 1, r = i >> 9;
            const u32x4 q4 = u32x4{tv[k], tv[k], tv[k], tv[k]};
            *reinterpret_cast<u32x4*>(&tab[r][m][c * 32 + 4 * g]) = q4;
            *reinterpret_cast<u32x4*>(&tab[r][m][c * 32 + 4 * (g + 4)]) = q4;
        }
    }
    if (l == 0) {
        meta[w][0] = nw > 0 ? qa : -1;
        meta[w][1] = nw > 0 ? qa + (na < nw ? 1 : 0) : -1;
    }

    __syncthreads();  // tables written
    if (nw > 0) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        int cq = qa;  // row-tile pair of the unit being multiplied
        int ckt = wu0 - qa * KT;
        // unit i from ring slot J; the refill is skipped past the run's end (the tail is not a
        // loop, so a conditional load there costs no drain)
        auto do_unit = [&](auto jc, int i, auto tailc) {
            constexpr int j = decltype(jc)::value;
            constexpr bool kTail = decltype(tailc)::value;
            const uint32_t tb = uint32_t((cq - q0) * 2) * (kTabDw * 4);
            const uint32_t lb0 = lane4 | tb, lb1 = lane4 | (tb + kTabDw * 4);
            const uint32_t d00 = rc[j][0][0], d01 = rc[j][0][1], d02 = rc[j][0][2];
            const uint32_t d10 = rc[j][1][0], d11 = rc[j][1][1], d12 = rc[j][1][2];
            u32x2 bw[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) bw[s] = u32x2{rb[j][s >> 1][2 * (s & 1)], rb[j][s >> 1][2 * (s & 1) + 1]};
#define SK_LOOK(Q, d0, d1, d2, lb) \
    (*reinterpret_cast<const uint32_t*>(tbase + code_addr<Q, 7>(d0, d1, d2, lb)))
#define SK_STEP(S)                                                                              \
    {                                                                                           \
        const u32x4 A0 = u32x4{SK_LOOK(4 * S + 0, d00, d01, d02, lb0),                          \
                               SK_LOOK(4 * S + 1, d00, d01, d02, lb0),                          \
                               SK_LOOK(4 * S + 2, d00, d01, d02, lb0),                          \
                               SK_LOOK(4 * S + 3, d00, d01, d02, lb0)};                         \
        const u32x4 A1 = u32x4{SK_LOOK(4 * S + 0, d10, d11, d12, lb1),                          \
                               SK_LOOK(4 * S + 1, d10, d11, d12, lb1),                          \
                               SK_LOOK(4 * S + 2, d10, d11, d12, lb1),                          \
                               SK_LOOK(4 * S + 3, d10, d11, d12, lb1)};                         \
        const uint32_t b0 = bw[S][0], b1 = bw[S][1];                                            \
        const u32x4 Bx = u32x4{__builtin_amdgcn_perm(b0, 0u, sel_e),                            \
                               __builtin_amdgcn_perm(b0, 0u, sel_o),                            \
                               __builtin_amdgcn_perm(b1, 0u, sel_e),                            \
                               __builtin_amdgcn_perm(b1, 0u, sel_o)};                           \
        acc[0] = mfma16x16x32(A0, Bx, acc[0]);                                                  \
        acc[1] = mfma16x16x32(A1, Bx, acc[1]);                                                  \
    }
            SK_STEP(0) SK_STEP(1) SK_STEP(2) SK_STEP(3)
#undef SK_STEP
#undef SK_LOOK
            // refill the slot once its words are used (the loads then reuse its registers);
            // kept here: left to itself the scheduler sinks the refills to the loop's end
            if constexpr (!kTail) load_unit(j);
            __builtin_amdgcn_sched_barrier(0);
            // the running sums go to the LDS slot of their row-tile pair after every unit, and
            // restart after the first pair's last unit: no branch in the loop (a branch makes
            // the compiler drain the whole ring at the loop head)
            const int seg = i < na ? 0 : 1;
            red[w][seg][0][l] = acc[0];
            red[w][seg][1][l] = acc[1];
            const bool restart = i + 1 == na;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[m][e] = restart ? 0.f : acc[m][e];
            if (++ckt == KT) {
                ckt = 0;
                ++cq;
            }
        };
        int i0 = 0;
        for (; i0 + kRing <= nw; i0 += kRing)
            sk_static_for<0, kRing>([&](auto jc) { do_unit(jc, i0 + decltype(jc)::value, std::false_type{}); });
        if (i0 < nw)
            sk_static_for<0, kRing>([&](auto jc) {
                if (i0 + decltype(jc)::value < nw) do_unit(jc, i0 + decltype(jc)::value, std::true_type{});
            });
    }
    __syncthreads();

    // ---- per row-tile pair: sum the waves that touched it, in wave order; thread (r, m, lane)
    if (tid < nq * 128) {
        const int r = tid >> 7, m = (tid >> 6) & 1, ln = tid & 63, q = q0 + r;
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int v = 0; v < kW; ++v) {
            const int va = meta[v][0], vb = meta[v][1];  // -1: no units
            if (q < va || q > vb) continue;
            sum += red[v][q == va ? 0 : 1][m][ln];
        }
        *reinterpret_cast<f32x4*>(a.part + size_t(q + b) * kSlot + (m * 64 + ln) * 4) = sum;
    }
}

// ---- finishing passes (after the projection's launch, so its slots are plain reads)

// sum of the slots of row-tile pair q, in workgroup order (empty ranges have no slot); w is the
// slot-relative word (tile m, lane, reg)
__device__ __forceinline__ float sk_slot_sum(const StreamKArgs& a, int G, int q, int w) {
    const int b0 = sk_owner(q * a.KT, a.U, G), b1 = sk_owner((q + 1) * a.KT - 1, a.U, G);
    float v = 0.f;
    for (int bb = b0; bb <= b1; ++bb)
        if (sk_start32(bb, a.U, G) != sk_start32(bb + 1, a.U, G)) v += a.part[size_t(q + bb) * kSlot + w];
    return v;
}

// gate/up: workgroup s finishes rotation span s (R = max(bi, 32) rows of the intermediate):
// a = SiLU(g s_g) (u s_u) . sign for the 8 operand rows, then x~ = H_bi(a) / sqrt(bi) in LDS
// (distances 1 .. bi/2 in that order, each pair (lo, hi) -> (lo + hi, lo - hi)), written in
// the unit-major binary16 layout the down projection reads.
__global__ void __launch_bounds__(1024) k_streamk_gu_fin(StreamKArgs a, int G) {
    __shared__ float buf[kSkinnyT * 1024];
    const int R = a.span, r0 = blockIdx.x * R, tid = threadIdx.x;
    // thread i < 8 R: pair q = (r0 + 32 j) / 32 with j = i / 256, lane ln, reg rg of its tile
    for (int i = tid; i < kSkinnyT * R; i += 1024) {
        const int q = r0 / kTileRows + (i >> 8), ln = (i >> 2) & 63, rg = i & 3;
        float g = sk_slot_sum(a, G, q, ln * 4 + rg);
        float u = sk_slot_sum(a, G, q, 256 + ln * 4 + rg);
        const int row = q * kTileRows + 2 * (4 * (ln >> 4) + rg) + (ln & 1), t = (ln & 15) >> 1;
        g *= h2f(a.mat[0].sc[row]);
        u *= h2f(a.mat[1].sc[row]);
        const float act = g / (1.f + expf(-g)) * u;
        const uint32_t sbit = a.sign_i && a.sign_i[row] < 0 ? 0x80000000u : 0u;
        buf[t * R + row - r0] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, act) ^ sbit);
    }
    __syncthreads();
    // (R and h are powers of two: shifts, no integer division)
    const int lr = 31 - __builtin_clz(R);
    for (int h = 1, lh = 0; h < a.bi; h <<= 1, ++lh) {
        for (int p = tid; p < kSkinnyT * R / 2; p += 1024) {
            const int t = p >> (lr - 1), k = p & (R / 2 - 1);
            const int i0 = (t << lr) + (((k >> lh) << (lh + 1)) | (k & (h - 1))), i1 = i0 + h;
            const float x0 = buf[i0], x1 = buf[i1];
            buf[i0] = x0 + x1;
            buf[i1] = x0 - x1;
        }
        __syncthreads();
    }
    for (int i = tid; i < kSkinnyT * R; i += 1024)
        a.ab_out[unit_major_index(i >> lr, r0 + (i & (R - 1)))] = uint16_t(f2h(buf[i] * a.norm_i));
}

// down: thread (q, tile m, lane, reg) sums the slots of q and scales into y
__global__ void __launch_bounds__(256) k_streamk_dn_fin(StreamKArgs a, int G) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.NQ * 512) return;
    const int q = i >> 9, m = (i >> 8) & 1, ln = (i >> 2) & 63, rg = i & 3;
    const int tile = 2 * q + m, t = (ln & 15) >> 1;
    if (tile >= a.MT || t >= a.T) return;
    const float v = sk_slot_sum(a, G, q, (m * 64 + ln) * 4 + rg);
    const int row = tile * kTileRows + 2 * (4 * (ln >> 4) + rg) + (ln & 1);
    a.y[size_t(t) * a.mat[0].N + row] = uint16_t(f2h(v * h2f(a.mat[0].sc[row])));
}

int streamk_grid(int nmat, int N, int K, int cus) {
    const int MT = N / kTileRows, KT = K / kTileCols;
    const int NQ = nmat == 2 ? MT : (MT + 1) / 2;
    const long long U = (long long)NQ * KT;
    if (MT < 1 || KT < 1 || U > (1 << 30)) return 0;
    // ranges of at most (kMaxQ - 1) KT + 1 units touch at most kMaxQ row-tile pairs, and their
    // wave runs (a sixteenth, rounded up) are no longer than KT
    const long long cap = (long long)(kMaxQ - 1) * KT + 1;
    long long g = cus > 0 ? cus : 1;
    if ((U + g - 1) / g > cap) g = (U + cap - 1) / cap;
    // (the combine passes index in 32 bits)
    return g > (1 << 20) || U * g >= (1ll << 31) ? 0 : int(g);
}

size_t streamk_part_floats(int nmat, int N, int K, int cus) {
    const int MT = N / kTileRows, NQ = nmat == 2 ? MT : (MT + 1) / 2;
    return size_t(NQ + streamk_grid(nmat, N, K, cus)) * kSlot;
}

hipError_t launch_streamk(const StreamKArgs& in, int cus, hipStream_t st) {
    StreamKArgs a = in;
    const int nmat = a.nmat;
    if (nmat == 1) a.mat[1] = a.mat[0];
    const int N = a.mat[0].N, K = a.mat[0].K;
    for (int m = 0; m < 2; ++m)
        if (!a.mat[m].codes || !a.mat[m].cb || !a.mat[m].sc || a.mat[m].N != N || a.mat[m].K != K)
            return hipErrorInvalidValue;
    if (!a.bx || !a.part || N % kTileRows || K % kTileCols || a.T < 1 || a.T > kSkinnyT)
        return hipErrorInvalidValue;
    if (nmat == 2) {
        // spans of max(bi, 32) rows (at most 1024: the finishing pass holds 8 x span floats)
        if (!a.ab_out || a.bi < 1 || a.bi > 1024 || (a.bi & (a.bi - 1)))
            return hipErrorInvalidValue;
        a.span = a.bi > kTileRows ? a.bi : kTileRows;
        if (N % a.span) return hipErrorInvalidValue;
    } else if (nmat != 1 || !a.y) {
        return hipErrorInvalidValue;
    }
    a.MT = N / kTileRows;
    a.KT = K / kTileCols;
    a.NQ = nmat == 2 ? a.MT : (a.MT + 1) / 2;
    a.U = a.NQ * a.KT;
    const int G = streamk_grid(nmat, N, K, cus);
    if (G < 1 || (long long)a.U * G >= (1ll << 31)) return hipErrorInvalidValue;
    if (nmat == 2) {
        hipLaunchKernelGGL(k_streamk<2>, dim3(G), dim3(kW * 64), 0, st, a);
        hipLaunchKernelGGL(k_streamk_gu_fin, dim3(N / a.span), dim3(1024), 0, st, a, G);
    } else {
        hipLaunchKernelGGL(k_streamk<1>, dim3(G), dim3(kW * 64), 0, st, a);
        hipLaunchKernelGGL(k_streamk_dn_fin, dim3((a.NQ * 512 + 255) / 256), dim3(256), 0, st, a, G);
    }
    return hipGetLastError();
}

}  // namespace vqmlp
