// fused.hip -- the whole T <= 8 MLP forward as one persistent kernel (gfx950).
//
//   x~ = R_H(x . s),  a = silu(W_gate x~) . (W_up x~) . sign_I,  y = W_down R_I(a)
//
// (model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP, token-mixer
// rotations, distilled weights": three-bit 2x64 vector tables for gate, up and down; online
// block-Hadamard rotations with seeded signs on the MLP inputs.)
//
// One workgroup of 16 waves per CU; workgroup b takes streaming items b, b + G, b + 2G, ... (G
// workgroups) after the input-rotation items r = b, b + G, ...:
//   R  rotate input columns [r*rc, (r+1)*rc) of x into x~ (binary16 pairs);
//   G  gate and up of one 32-row tile over all of H (the matrix-core product of the skinny
//      kernel: lane-private LDS codebooks, register code ring), epilogue silu(g) u sign;
//   D  down projection of two 32-row tiles over one K slice of 16 * TPW tiles of I.
// Work that needs several items is done right after one item of the set:
//   F  one G tile of each rotation unit (max(bi, 32) rows; all tiles of a unit are processed
//      in the same round by different workgroups) rotates the unit's a into the binary16 down
//      operand once the other tiles' values are in;
//   Y  the D item of the last K slice of a row pair sums the slices, scales and writes y.
// Every hand-off between items goes through global memory as 64-bit words {32 data bits, tag},
// tag = call epoch + 1: the reader checks each word itself and the writer never waits for its
// stores.  On this GPU a wave's loads complete in order and any wait for a store also waits for
// every older load, so a flag protocol (writer: wait for the stores, then raise a flag; reader:
// see the flag, then load) would cost two more memory round trips per hand-off, each behind
// the wave's code prefetch.  Rotations run in registers, one operand row per wave.
// Every wait is bounded by spin_limit; a wait that runs out sets a bit in the error word and
// the kernel finishes with wrong values instead of hanging.  No item waits for a later item of
// its own workgroup and the grid is one workgroup per CU, so every wait ends.
#include "device.h"
#include "internal.h"

namespace vqmlp {

namespace {

constexpr int kW = kSkinnyWaves;   // 16 waves
constexpr int kTab = 64 * 32;      // dwords of one lane-private table set (one tile, one matrix)
constexpr int kKindG = 0, kKindD = 1, kKindNone = 2;

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A 64-bit load that may hit caches (it can return an older value of the word; tagged words
// make that visible to the reader).
__device__ __forceinline__ uint64_t ld_cached64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_relaxed64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void note_error(uint32_t* ctl, uint32_t bit) {
    __hip_atomic_fetch_or(ctl + kCtlError, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float dpp_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                              0xF, 0xF, false));
}

// Sum of the 16 floats p[0], p[stride], ..., p[15 stride] in a fixed pairwise order.
__device__ __forceinline__ float sum16(const float* p, int stride) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = p[i * stride];
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; i += 2 * h) v[i] += v[i + h];
    return v[0];
}

constexpr int kRotVals = 4;  // values per lane of a rotated row (rows of up to 256 columns)

// Walsh-Hadamard butterflies (Sylvester order, distances 1 .. b/2) over one row held by a wave:
// value e < ne of lane l is column 64 e + l, or column l % 32 of a 32-column row (both halves
// of the wave then hold it).  Distances below 64 pair lanes l and l ^ h; larger ones pair
// values e and e ^ (h / 64) of one lane.
__device__ __forceinline__ void wave_fwht(float (&v)[kRotVals], int ne, int b, int l) {
    for (int h = 1; h < b && h < 64; h <<= 1) {
        const bool upper = (l & h) != 0;
#pragma unroll
        for (int e = 0; e < kRotVals; ++e)
            if (e < ne) {
                const float p = __shfl_xor(v[e], h);
                v[e] = upper ? p - v[e] : v[e] + p;
            }
    }
#pragma unroll
    for (int d = 1; d < kRotVals; d <<= 1)
        if (64 * d < b) {
#pragma unroll
            for (int e = 0; e < kRotVals; ++e)
                if (!(e & d) && (e | d) < ne) {
                    const float x0 = v[e], x1 = v[e | d];
                    v[e] = x0 + x1;
                    v[e | d] = x0 - x1;
                }
        }
}

// A streaming item, decoded from its queue index (all fields uniform).
struct Item {
    int kind;   // kKindG, kKindD or kKindNone
    int id;     // G: row tile m; D: row pair q
    int sl;     // K slice (0 for G)
    int t0, t1; // row tiles of the two operand slots
    int KT;     // K tiles of the matrix
};

}  // namespace

template <int TPW>
__global__ void __launch_bounds__(kW * 64, 1) k_fused(FusedArgs a) {
    constexpr int D = TPW;  // ring slots: slot t always holds tile t of some item
    // Prefetch distance in tiles.  Code words are requested P tiles before their use, not a whole
    // item ahead: the deeper the queue of streaming loads, the longer every other load of the
    // workgroup (flags, hand-off words) waits behind it.
    constexpr int P = TPW < 2 ? TPW : 2;
    constexpr int SWT = kW * TPW;  // K tiles per slice
    constexpr int BROW = SWT * kTileCols + 16;  // padded row of the activation operand
    // One LDS block with the lookup tables at address 0: a lookup address is then the code and
    // lane bits alone, with no base to add.
    constexpr int kOffRed = 2 * 2 * kTab * 4;
    constexpr int kOffB = kOffRed + kW * 2 * 64 * 16;
    constexpr int kOffEsc = kOffB + kSkinnyT * BROW * 2;
    constexpr int kOffEsg = kOffEsc + 4 * 2 * 32 * 4;
    constexpr int kOffOk = kOffEsg + 4 * 32 * 4;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kOffOk + 16];
    auto& tab = *reinterpret_cast<uint32_t (*)[2][2][kTab]>(lds);          // [buffer][slot][table]
    auto& red = *reinterpret_cast<f32x4 (*)[kW][2][64]>(lds + kOffRed);   // partials, scratch
    auto& bsh = *reinterpret_cast<uint16_t (*)[kSkinnyT][BROW]>(lds + kOffB);  // activations
    auto& esc = *reinterpret_cast<float (*)[4][2][32]>(lds + kOffEsc);    // row scales
    auto& esg = *reinterpret_cast<uint32_t (*)[4][32]>(lds + kOffEsg);    // sign bits
    int& qslot = *reinterpret_cast<int*>(lds + kOffOk);                    // item after next

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, I = a.I, T = a.T;
    const int MTh = H / kTileRows, KTh = H / kTileCols, KTi = I / kTileCols;
    uint32_t* const ctl = a.ctl;
    const uint32_t tag = ld_relaxed(ctl + kCtlEpoch) + 1u;
    // The operand hand-offs alternate between two buffers by call parity: a cached line of the
    // previous call then never shadows this call's words (and the tags catch older ones).
    uint64_t* const xbp = a.xb + (tag & 1u) * size_t(kSkinnyT) * (H / 2);
    uint64_t* const abp = a.ab + (tag & 1u) * size_t(kSkinnyT) * (I / 2);
    const unsigned limit = a.spin_limit;

    auto decode = [&](int u) -> Item {
        Item it;
        it.sl = 0;
        if (u < a.n_r || u >= a.total) {
            it.kind = kKindNone;
            it.id = 0;
            it.t0 = it.t1 = 0;
            it.KT = KTh;
        } else if (u < a.n_r + a.n_g) {
            it.kind = kKindG;
            it.id = u - a.n_r;
            it.t0 = it.t1 = it.id;
            it.KT = KTh;
        } else {
            const int v = u - a.n_r - a.n_g;
            it.kind = kKindD;
            it.sl = v / a.nqd;
            it.id = v % a.nqd;
            it.t0 = min(2 * it.id, MTh - 1);
            it.t1 = min(2 * it.id + 1, MTh - 1);
            it.KT = KTi;
        }
        return it;
    };
    // this wave's K tiles of an item: [kt0, kt0 + ntile), loads clamped to last_kt
    auto wave_tiles = [&](const Item& it, int& kt0, int& ntile, int& last_kt) {
        kt0 = it.sl * SWT + w * TPW;
        ntile = it.KT - kt0;
        ntile = ntile < TPW ? (ntile > 0 ? ntile : 0) : TPW;
        last_kt = kt0 + (ntile > 0 ? ntile : 1) - 1;
        last_kt = last_kt < it.KT ? last_kt : it.KT - 1;
    };
    auto tile_word = [&](const Item& it, int m, int kt) -> const uint32_t* {
        const uint8_t* base = it.kind == kKindD ? a.down.codes : (m ? a.up.codes : a.gate.codes);
        const int mt = m ? it.t1 : it.t0;
        return reinterpret_cast<const uint32_t*>(base + (size_t(mt) * it.KT + kt) * kTileBytes) +
               3 * l;
    };

    // ---- per-item table operands: threads 0..511 one codebook word each (slot, group, entry);
    // waves 8 and 9 the row scales of slot 0 and 1; wave 10 the signs
    const int cb_m = (w >> 2) & 1, cb_g = w & 3, cb_c = l;  // slot and group uniform per wave
    // one register per thread: a codebook word (waves 0-7), a row scale (waves 8, 9) or a sign
    // (wave 10)
    // One dword per thread, loaded with no branch around the load (a load under a branch makes
    // the next one wait for every older load, the code prefetch included): waves 0-7 a codebook
    // word, waves 8 and 9 the dword holding their lane's row scale, wave 10 the dword holding
    // its lane's sign; the other waves load a codebook word they ignore.
    auto load_tab = [&](const Item& it) -> uint32_t {
        const bool dn = it.kind == kKindD;
        const int mt = cb_m ? it.t1 : it.t0, sm = w & 1, r32 = l & 31;
        const uint32_t* cbp =
            (dn ? a.down.cb : (cb_m ? a.up.cb : a.gate.cb)) + size_t(mt * 4 + cb_g) * 64 + cb_c;
        const uint16_t* scb = dn ? a.down.sc : (sm ? a.up.sc : a.gate.sc);
        const uint32_t* scp = reinterpret_cast<const uint32_t*>(
            scb + (sm ? it.t1 : it.t0) * kTileRows + (r32 & ~1));
        // the sign belongs to rows of I: only a gate/up item's row tile indexes it (a down
        // item's tiles are rows of H, which may run past I; it reads tile 0 and ignores it)
        const int8_t* sgb = a.sign_i ? a.sign_i : reinterpret_cast<const int8_t*>(a.gate.sc);
        const int sgt = it.kind == kKindG ? it.t0 : 0;
        const uint32_t* sgp =
            reinterpret_cast<const uint32_t*>(sgb + sgt * kTileRows + (r32 & ~3));
        const uint32_t* p = (w == 8 || w == 9) ? scp : (w == 10 ? sgp : cbp);
        return *p;
    };
    // signed: the item is a gate/up item and the intermediate rotation has signs
    auto store_tab = [&](int buf, int eb, uint32_t v, bool signed_) {
        if (w < 8) {
            const u32x4 q = u32x4{v, v, v, v};
            *reinterpret_cast<u32x4*>(&tab[buf][cb_m][cb_c * 32 + 4 * cb_g]) = q;
            *reinterpret_cast<u32x4*>(&tab[buf][cb_m][cb_c * 32 + 4 * (cb_g + 4)]) = q;
        } else if ((w == 8 || w == 9) && l < 32) {
            esc[eb][w - 8][l] = h2f(v >> (16 * (l & 1)));
        } else if (w == 10 && l < 32) {
            const uint32_t byte = (v >> (8 * (l & 3))) & 0xFFu;
            esg[eb][l] = signed_ ? (byte >> 7) << 31 : 0u;
        }
    };

    // ---- rotations: wave t < 8 rotates operand row t in registers (value e of lane l is column
    // 64 e + l of the range, or column l % 32 of a 32-column range); even lanes store pairs
    auto store_pairs = [&](uint64_t* dst, const float (&v)[kRotVals], int ne, int n, float norm) {
#pragma unroll
        for (int e = 0; e < kRotVals; ++e)
            if (e < ne) {
                const float mine = v[e] * norm, next = dpp_xor1(mine);
                const int c = n >= 64 ? 64 * e + l : l;
                if (!(l & 1) && c < n)
                    st_relaxed64(dst + c / 2, (uint64_t(tag) << 32) | f2h(mine) | (f2h(next) << 16));
            }
    };
    // input rotation item r: columns [r*rc, (r+1)*rc) of x . s . sign, all 8 operand rows
    auto rotate_in = [&](int r) {
        const int rc = a.rc, c0 = r * rc, ne = rc >= 64 ? rc / 64 : 1;
        if (w < kSkinnyT) {
            float v[kRotVals];
#pragma unroll
            for (int e = 0; e < kRotVals; ++e) {
                v[e] = 0.f;
                const int col = c0 + (rc >= 64 ? 64 * e + l : (l & 31));
                if (e < ne && w < T) {
                    v[e] = h2f(a.x[size_t(w) * H + col]) * h2f(a.s[col]);
                    if (a.sign_h && a.sign_h[col] < 0) v[e] = -v[e];
                }
            }
            wave_fwht(v, ne, a.bh, l);
            store_pairs(xbp + size_t(w) * (H / 2) + c0 / 2, v, ne, rc, a.norm_h);
        }
    };

    // ---- F: rotate rotation unit u of a into the binary16 down operand
    auto job_rotate_mid = [&](int u) {
        const int fu = a.fu, r0 = u * fu, ne = fu >= 64 ? fu / 64 : 1;
        if (w < kSkinnyT) {
            const uint64_t* src = a.act + size_t(w) * I + r0;
            uint64_t q[kRotVals];
#pragma unroll
            for (int e = 0; e < kRotVals; ++e)
                q[e] = e < ne ? ld_relaxed64(src + (fu >= 64 ? 64 * e + l : (l & 31))) : 0;
            // the other tiles of the unit may still be on their way: wait for every word's tag
            for (unsigned n = 0;; ++n) {
                bool ready = true;
#pragma unroll
                for (int e = 0; e < kRotVals; ++e)
                    if (e < ne && uint32_t(q[e] >> 32) != tag) ready = false;
                if (ready) break;
                if (n >= limit) {
                    note_error(ctl, 2u);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
#pragma unroll
                for (int e = 0; e < kRotVals; ++e)
                    if (e < ne && uint32_t(q[e] >> 32) != tag)
                        q[e] = ld_relaxed64(src + (fu >= 64 ? 64 * e + l : (l & 31)));
            }
            float v[kRotVals];
#pragma unroll
            for (int e = 0; e < kRotVals; ++e) v[e] = __builtin_bit_cast(float, uint32_t(q[e]));
            wave_fwht(v, ne, a.bi, l);
            store_pairs(abp + size_t(w) * (I / 2) + r0 / 2, v, ne, fu, a.norm_i);
        }
    };

    // ---- Y: y rows of pair q = sum over slices of the tagged partials, scaled
    auto job_reduce_y = [&](int q) {
        if (tid < 512) {
            const int t = tid >> 6, row = 64 * q + (tid & 63);
            if (t < T && row < H) {
                float sum = 0.f;
                bool good = true;
                for (int sl = 0; sl < a.nsl; ++sl) {
                    const uint64_t* p = a.part + (size_t(sl) * kSkinnyT + t) * H + row;
                    uint64_t v = ld_relaxed64(p);
                    for (unsigned n = 0; uint32_t(v >> 32) != tag; ++n) {
                        if (n >= limit) {
                            good = false;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                        v = ld_relaxed64(p);
                    }
                    sum += __builtin_bit_cast(float, uint32_t(v));
                }
                if (!good) note_error(ctl, 4u);
                a.y[size_t(t) * H + row] = (uint16_t)f2h(sum * h2f(a.down.sc[row]));
            }
        }
    };

    // ================================================================ start: input rotations
    const int G = gridDim.x, b = blockIdx.x;
    for (int r = b; r < a.n_r; r += G) rotate_in(r);

    // operand selectors: lane l holds column n = l%16 = 2*tok + cp of B
    const int n16 = l & 15, tok = n16 >> 1, cp = n16 & 1;
    const uint32_t sel_e = cp ? 0x05040C0Cu : 0x0C0C0504u;
    const uint32_t sel_o = cp ? 0x07060C0Cu : 0x0C0C0706u;
    const uint32_t lane4 = uint32_t(l & 31) << 2;
    const char* tbase = reinterpret_cast<const char*>(&tab[0][0][0]);
    // this lane's activation words: token tok, columns 16 s + 4 (l / 16) of each tile
    const uint16_t* bl = &bsh[tok][w * TPW * kTileCols + 4 * (l >> 4)];

    // streaming items b, b + G, b + 2G, ... of the gate/up items followed by the down items
    int cur_u = a.n_r + b;
    {
        const Item c = decode(cur_u);
        store_tab(0, 0, load_tab(c), c.kind == kKindG && a.sign_i);
    }
    uint32_t ring[D][2][3];
    {
        const Item c = decode(cur_u);
        int kt0, ntile, last_kt;
        wave_tiles(c, kt0, ntile, last_kt);
        if (c.kind != kKindNone) {
#pragma unroll
            for (int t = 0; t < P; ++t)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int kt = kt0 + t < last_kt ? kt0 + t : last_kt;
                    const uint32_t* p = tile_word(c, m, kt);
                    ring[t][m][0] = p[0];
                    ring[t][m][1] = p[1];
                    ring[t][m][2] = p[2];
                }
        }
    }
    int prev_u = -1;   // the previous streaming item
    int bstate = -1;   // activation slice in bsh: 0 = x~, 1 + s = rotated a slice s
    const int tpu = a.fu / kTileRows;  // gate/up tiles per rotation unit

    // Items after the first two rounds come from the queue (a.dyn) or round-robin.  The queue
    // is read one item ahead of the next one, whose codes are prefetched during this item.
    int nxt_u = a.n_r + b + G;
    for (int j = 0;; ++j) {
        const int buf = j & 1;
        __syncthreads();  // (A) tables of cur and partials of prev are complete
        if (j > 0) nxt_u = a.dyn ? min(a.n_r + 2 * G + qslot, a.total) : cur_u + G;

        // (C) epilogue of the previous item: reduce the 16 waves' partials
        int job = -1;  // F: rotation unit; Y: (1 << 30) | row pair
        if (prev_u >= 0) {
            const Item prev = decode(prev_u);
            const int eb = (j - 1) & 3;
            if (prev.kind == kKindG) {
                // Thread tid < 256 sums the 16 waves' partials of accumulator element
                // e_r = tid % 4 of lane e_l = tid / 4 (both matrices).  Float 4 e_l + e_r of a
                // wave's block is tid, so a wave's 64 reads of one block fall in 64 consecutive
                // words: every bank once per half-wave.
                const int e_l = tid >> 2, e_r = tid & 3;
                if (tid < 256) {
                    const float* rf = reinterpret_cast<const float*>(&red[0][0][0]) + e_l * 4 + e_r;
                    float g = sum16(rf, 512), u = sum16(rf + 256, 512);
                    const int rl = 2 * (4 * (e_l >> 4) + e_r) + (e_l & 1), t = (e_l & 15) >> 1;
                    g *= esc[eb][0][rl];
                    u *= esc[eb][1][rl];
                    const float act = silu(g) * u;
                    const uint32_t bits = __builtin_bit_cast(uint32_t, act) ^ esg[eb][rl];
                    st_relaxed64(a.act + size_t(t) * I + prev.id * kTileRows + rl,
                                 (uint64_t(tag) << 32) | bits);
                }
                // One tile of each rotation unit rotates the whole unit once the others' values
                // are in.  Round-robin order: which tile is hashed from the unit, so that the
                // rotations do not all fall to the same workgroups.  Queue order: the unit's last
                // tile, so the rotation only ever waits for tiles handed out before it.
                const int unit = prev.id / tpu;
                const int owner = a.dyn ? tpu - 1 : int((unit ^ (unit >> 2) ^ (unit >> 5)) % tpu);
                if (prev.id % tpu == owner) job = unit;
            } else {
                // Thread tid < 512 sums the 16 waves' partials of element e_r of lane e_l of
                // operand slot mm (bank tid % 32, as in the gate/up epilogue).
                const int mm = tid >> 8, e_l = (tid >> 2) & 63, e_r = tid & 3;
                const int tile = 2 * prev.id + mm;
                if (tid < 512 && tile < MTh) {
                    const float* rf =
                        reinterpret_cast<const float*>(&red[0][0][0]) + mm * 256 + e_l * 4 + e_r;
                    const float v = sum16(rf, 512);
                    const int rl = 2 * (4 * (e_l >> 4) + e_r) + (e_l & 1), t = (e_l & 15) >> 1;
                    const int row = tile * kTileRows + rl;
                    if (a.nsl == 1) {
                        if (t < T) a.y[size_t(t) * H + row] = (uint16_t)f2h(v * esc[eb][mm][rl]);
                    } else {
                        st_relaxed64(a.part + (size_t(prev.sl) * kSkinnyT + t) * H + row,
                                     (uint64_t(tag) << 32) | __builtin_bit_cast(uint32_t, v));
                    }
                }
                // the last slice of a row pair sums the slices
                if (a.nsl > 1 && prev.sl == a.nsl - 1) job = (1 << 30) | prev.id;
            }
        }
        __syncthreads();  // (B) partials consumed: red is free
        // (D) the rotation unit or row pair that this epilogue completed (waves 0-7).  No barrier
        // after it, so the other waves start the next item at once: the jobs touch no LDS, and
        // what this iteration writes to LDS from here on (the idle table buffer, scale slots two
        // items ahead, red and the queue slot after barrier (B), each wave's own activation
        // columns) is read by no wave before the next barrier (A).
        if (job >= 0) {
            if (job >> 30)
                job_reduce_y(job & ((1 << 30) - 1));
            else
                job_rotate_mid(job);
        }
        if (cur_u >= a.total) break;

        // (F) table operands of the next item (written after this item's products)
        const Item nit = decode(nxt_u);
        const uint32_t tv_next = load_tab(nit);
        const bool sg_next = nit.kind == kKindG && a.sign_i;
        // the queue slot after next; its value is first used after this item's products, so the
        // wait for it does not hold up their code loads
        uint32_t qv = uint32_t(a.total - a.n_r - 2 * G);
        if (a.dyn && tid == 0 && nxt_u < a.total)
            qv = __hip_atomic_fetch_add(ctl + kCtlQueue, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);

        // (G) activation operand of this item: one K slice of x~ or of the rotated a, 8 rows
        {
            const Item cur = decode(cur_u);
            const int want = cur.kind == kKindG ? 0 : 1 + cur.sl;
            if (want != bstate) {
                // Each wave waits for, and loads, only the columns of its own tiles: a wave whose
                // inputs are ready starts while the others still wait.  The operand words carry
                // the call's tag; a word whose tag is not yet this call's is read again.
                constexpr int wcols = TPW * kTileCols;
                {
                    constexpr int kPairs = wcols / 2;                 // pairs per operand row
                    constexpr int kM = (kPairs + 63) / 64;            // pairs per lane and row
                    const int c0 = cur.sl * SWT * kTileCols + w * wcols;
                    const int K = cur.kind == kKindG ? H : I;
                    // lane l holds pairs l + 64 m of every row; pairs past K multiply zero (their
                    // code loads are clamped)
                    const uint64_t* src = (cur.kind == kKindG ? xbp : abp) + c0 / 2 + l;
                    const int npair = min(kPairs, (K - c0) / 2);
                    uint64_t q[kSkinnyT][kM];
                    // first through the caches (the operand is shared by many workgroups), then
                    // coherently for the words that are not yet this call's
#pragma unroll
                    for (int t = 0; t < kSkinnyT; ++t)
#pragma unroll
                        for (int m = 0; m < kM; ++m)
                            q[t][m] = l + 64 * m < npair
                                          ? ld_cached64(src + size_t(t) * (K / 2) + 64 * m)
                                          : uint64_t(tag) << 32;
                    auto fetch = [&]() {
#pragma unroll
                        for (int t = 0; t < kSkinnyT; ++t)
#pragma unroll
                            for (int m = 0; m < kM; ++m)
                                if (uint32_t(q[t][m] >> 32) != tag)
                                    q[t][m] = ld_relaxed64(src + size_t(t) * (K / 2) + 64 * m);
                    };
                    for (unsigned n = 0;; ++n) {
                        bool ready = true;
#pragma unroll
                        for (int t = 0; t < kSkinnyT; ++t)
#pragma unroll
                            for (int m = 0; m < kM; ++m)
                                if (uint32_t(q[t][m] >> 32) != tag) ready = false;
                        if (ready) break;
                        if (n >= limit) {
                            note_error(ctl, 1u);
                            break;
                        }
                        fetch();
                        __builtin_amdgcn_s_sleep(2);
                    }
#pragma unroll
                    for (int t = 0; t < kSkinnyT; ++t)
#pragma unroll
                        for (int m = 0; m < kM; ++m)
                            if (l + 64 * m < kPairs)
                                *reinterpret_cast<uint32_t*>(&bsh[t][w * wcols + 2 * (l + 64 * m)]) =
                                    uint32_t(q[t][m]);
}
                bstate = want;
            }
        }

        // (H) the products; the code ring streams on into the next item's tiles (or reloads
        // this item's own when there is none)
        {
            const bool has_next = nxt_u < a.total;  // uniform
            const Item pit = decode(has_next ? nxt_u : cur_u);
            int nkt0, nntile, nlast_kt;
            wave_tiles(pit, nkt0, nntile, nlast_kt);
            const uint8_t* nbase0 = (pit.kind == kKindD ? a.down.codes : a.gate.codes) +
                                    size_t(pit.t0) * pit.KT * kTileBytes;
            const uint8_t* nbase1 = (pit.kind == kKindD ? a.down.codes : a.up.codes) +
                                    size_t(pit.t1) * pit.KT * kTileBytes;
            const Item cit = decode(cur_u);
            int ckt0, cntile, clast_kt;
            wave_tiles(cit, ckt0, cntile, clast_kt);
            const uint8_t* cbase0 = (cit.kind == kKindD ? a.down.codes : a.gate.codes) +
                                    size_t(cit.t0) * cit.KT * kTileBytes;
            const uint8_t* cbase1 = (cit.kind == kKindD ? a.down.codes : a.up.codes) +
                                    size_t(cit.t1) * cit.KT * kTileBytes;
            uint32_t laneb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) laneb[m] = lane4 | uint32_t((buf * 2 + m) * kTab * 4);
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
            // slot t + P: tile t + P of this item, or of the next one past the end.  With no
            // next item the load repeats tile t, just read and still in the on-die cache: the
            // refill stays unconditional without fetching again a tile that left the cache.
            auto refill = [&](const int t) {
                const int tt = (t + P) % TPW;
                const bool own = t + P < TPW || !has_next;
                int kt = t + P < TPW ? ckt0 + tt : (has_next ? nkt0 + tt : ckt0 + t);
                const int lim = own ? clast_kt : nlast_kt;
                kt = kt < lim ? kt : lim;
                const uint32_t* p0 = reinterpret_cast<const uint32_t*>(
                                         (own ? cbase0 : nbase0) + size_t(kt) * kTileBytes) + 3 * l;
                const uint32_t* p1 = reinterpret_cast<const uint32_t*>(
                                         (own ? cbase1 : nbase1) + size_t(kt) * kTileBytes) + 3 * l;
                ring[tt][0][0] = p0[0];
                ring[tt][0][1] = p0[1];
                ring[tt][0][2] = p0[2];
                ring[tt][1][0] = p1[0];
                ring[tt][1][1] = p1[1];
                ring[tt][1][2] = p1[2];
            };
            if (cntile == 0) {
                // no tile of this item (the last K slice is short): only the refills that
                // fetch the next item's first tiles
#pragma unroll
                for (int t = TPW - P; t < TPW; ++t)
                    if (t >= 0) refill(t);
            } else {
                u32x4 A[2][2];
                look(ring[0], 0, A[0]);
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int cp0 = (4 * t + s) & 1, cp1 = cp0 ^ 1;
                        const u32x2 bv = *reinterpret_cast<const u32x2*>(bl + t * kTileCols + 16 * s);
                        if (s < 3)
                            look(ring[t % D], s + 1, A[cp1]);
                        else if (t + 1 < TPW)
                            look(ring[(t + 1) % D], 0, A[cp1]);
                        if (s == 2) {
                            refill(t);
                            // keep each refill where it is, one item ahead of its use
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        const uint32_t b0 = bv[0], b1 = bv[1];
                        const u32x4 Bx = u32x4{__builtin_amdgcn_perm(b0, 0u, sel_e),
                                               __builtin_amdgcn_perm(b0, 0u, sel_o),
                                               __builtin_amdgcn_perm(b1, 0u, sel_e),
                                               __builtin_amdgcn_perm(b1, 0u, sel_o)};
                        acc[0] = mfma16x16x32(A[cp0][0], Bx, acc[0]);
                        acc[1] = mfma16x16x32(A[cp0][1], Bx, acc[1]);
                    }
                }
            }
            // (I) next item's tables into the idle buffers, this item's partials
            store_tab(buf ^ 1, (j + 1) & 3, tv_next, sg_next);
            red[w][0][l] = acc[0];
            red[w][1][l] = acc[1];
            if (tid == 0) qslot = int(qv);
        }
        prev_u = cur_u;
        cur_u = nxt_u;
    }

    // ================================================================ exit: the last workgroup
    // advances the epoch for the next call (flags and tags of this call then go stale)
    __syncthreads();
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(ctl + kCtlExit, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done + 1u == gridDim.x) {
            ctl[kCtlExit] = 0u;
            ctl[kCtlQueue] = 0u;
            ctl[kCtlEpoch] = tag;
        }
    }
}

int fused_tpw(int H) {
    const int KT = H / kTileCols;
    const int tpw = (KT + kW - 1) / kW;
    return tpw >= 1 && tpw <= kSkinnyMaxTPW ? tpw : 0;
}

hipError_t launch_fused(const FusedArgs& a, int tpw, int grid, hipStream_t st) {
    if (!a.y || !a.ctl || grid < 1 || (a.nsl > 1 && !a.part) || a.fu < kTileRows ||
        a.fu > 64 * kRotVals || a.rc > 64 * kRotVals || a.n_r > kW * 64 || a.T < 1 ||
        a.T > kSkinnyT)
        return hipErrorInvalidValue;
    if (!a.x || !a.s || !a.xb || !a.act || !a.ab) return hipErrorInvalidValue;
#define VQ_CASE(TP)                                                               \
    if (tpw == TP) {                                                              \
        hipLaunchKernelGGL((k_fused<TP>), dim3(grid), dim3(kW * 64), 0, st, a);   \
        return hipGetLastError();                                                 \
    }
    VQ_CASE(1) VQ_CASE(2) VQ_CASE(3) VQ_CASE(4) VQ_CASE(5)
#undef VQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace vqmlp
