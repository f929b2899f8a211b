// kernels.hip -- HIP kernels for gfx950 (CDNA4): block-Hadamard rotation and dequantisation.
//
// Weight format (model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit
// MLP, token-mixer rotations, distilled weights"): W[r][j] = cb[r/8][code[r/2][j]][r%2] * sc[r],
// six-bit codes into 64 two-component binary16 centroids per group of 8 output rows.
#include "device.h"
#include "internal.h"

namespace vqmlp {

// ==================================================================== dequantisation (test hook)

template <int Q>
__device__ __forceinline__ void dequant_one(const VQ3View& m, float* w, int pair, int col_base,
                                            int l, uint32_t d0, uint32_t d1, uint32_t d2, float s0,
                                            float s1) {
    const uint32_t code = code_of<Q>(d0, d1, d2);
    const int col = col_base + 16 * (Q / 4) + 4 * (l / 16) + (Q % 4);
    const uint32_t e = m.cb[(pair / 4) * 64 + code];
    w[size_t(2 * pair) * m.K + col] = h2f(e & 0xFFFFu) * s0;
    w[size_t(2 * pair + 1) * m.K + col] = h2f(e >> 16) * s1;
}

template <int... Qs>
__device__ __forceinline__ void dequant_all(const VQ3View& m, float* w, int pair, int col_base,
                                            int l, uint32_t d0, uint32_t d1, uint32_t d2, float s0,
                                            float s1, std::integer_sequence<int, Qs...>) {
    (dequant_one<Qs>(m, w, pair, col_base, l, d0, d1, d2, s0, s1), ...);
}

__global__ void __launch_bounds__(64) k_dequant(VQ3View m, float* w) {
    const int KT = m.K / kTileCols;
    const int tile = blockIdx.x;
    const int mt = tile / KT, kt = tile % KT, l = threadIdx.x;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(m.codes + size_t(tile) * kTileBytes) + 3 * l;
    const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
    const int pair = mt * kTilePairs + (l % 16);
    const float s0 = h2f(m.sc[2 * pair]), s1 = h2f(m.sc[2 * pair + 1]);
    dequant_all(m, w, pair, kt * kTileCols, l, d0, d1, d2, s0, s1,
                std::make_integer_sequence<int, 16>{});
}

hipError_t launch_dequant(const VQ3View& m, float* w, hipStream_t s) {
    const int tiles = (m.N / kTileRows) * (m.K / kTileCols);
    hipLaunchKernelGGL(k_dequant, dim3(tiles), dim3(64), 0, s, m, w);
    return hipGetLastError();
}

// ==================================================================== block-Hadamard rotation
//
// out = (I (x) H_b / sqrt(b)) diag(sign) (x . s), H_b Sylvester-ordered, evaluated with the
// in-place butterfly (a, c) -> (a + c, a - c) over strides 1, 2, 4, ..., b/2, in FP32.
// One workgroup rotates one block of b columns for 8 rows.

// One wave rotates one chunk of 64 * NE columns of one row (one block when b >= 64, 64 / b blocks
// otherwise), in registers: value e of lane l is column c0 + 64 e + l.  Butterfly distances
// below 64 pair lanes (cross-lane shuffles), larger ones pair values of a lane.
template <int NE>
__global__ void __launch_bounds__(256) k_rotate(int T, int rows, int n, int b, const void* x,
                                                int x_is_f32, const uint16_t* s,
                                                const int8_t* sign, void* out, int mode,
                                                float norm) {
    const int l = threadIdx.x & 63;
    const int chunks = (n + 64 * NE - 1) / (64 * NE);
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= rows * chunks) return;
    const int t = wv / chunks, c0 = (wv % chunks) * 64 * NE;
    float v[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int col = c0 + 64 * e + l;
        float u = 0.f;
        if (col < n && t < T) {
            const size_t idx = size_t(t) * n + col;
            u = x_is_f32 ? static_cast<const float*>(x)[idx]
                         : h2f(static_cast<const uint16_t*>(x)[idx]);
            if (s) u *= h2f(s[col]);
            if (sign && sign[col] < 0) u = -u;
        }
        v[e] = u;
    }
    for (int h = 1; h < b && h < 64; h <<= 1) {
        const bool upper = (l & h) != 0;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const float p = __shfl_xor(v[e], h);
            v[e] = upper ? p - v[e] : v[e] + p;
        }
    }
#pragma unroll
    for (int d = 1; d < NE; d <<= 1)
        if (64 * d < b) {
#pragma unroll
            for (int e = 0; e < NE; ++e)
                if (!(e & d)) {
                    const float x0 = v[e], x1 = v[e | d];
                    v[e] = x0 + x1;
                    v[e | d] = x0 - x1;
                }
        }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int col = c0 + 64 * e + l;
        if (col >= n) continue;
        const size_t idx = size_t(t) * n + col;
        const float r = v[e] * norm;
        if (mode == 0)
            static_cast<float*>(out)[idx] = r;
        else
            static_cast<uint16_t*>(out)[idx] = (uint16_t)f2h(r);
    }
}

// The same rotation with V consecutive columns per lane (a wave covers 64 V columns of one row):
// every load and store is a 16-byte vector access, butterflies of distance below V stay in the
// lane and the others pair lane l with lane l ^ (h / V).  Needs n to be a multiple of 64 V.
template <int V>
__global__ void __launch_bounds__(256) k_rotate_v(int T, int rows, int n, int b, const void* x,
                                                  int x_is_f32, const uint16_t* s,
                                                  const int8_t* sign, void* out, int mode,
                                                  float norm) {
    static_assert(V == 8 || V == 16, "16-byte accesses");
    const int l = threadIdx.x & 63;
    const int chunks = n / (64 * V);
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= rows * chunks) return;
    const int t = wv / chunks, col = (wv % chunks) * 64 * V + V * l;
    float v[V];
    if (t < T) {
        const size_t idx = size_t(t) * n + col;
        if (x_is_f32) {
            const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + idx);
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const f32x4 u = p[q];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * q + e] = u[e];
            }
        } else {
            const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + idx);
#pragma unroll
            for (int q = 0; q < V / 8; ++q) {
                const u32x4 u = p[q];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[8 * q + e] = h2f(u[e / 2] >> (16 * (e & 1)));
            }
        }
        if (s) {
            const u32x4* p = reinterpret_cast<const u32x4*>(s + col);
#pragma unroll
            for (int q = 0; q < V / 8; ++q) {
                const u32x4 u = p[q];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[8 * q + e] *= h2f(u[e / 2] >> (16 * (e & 1)));
            }
        }
        if (sign) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(sign + col);
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const uint32_t u = p[q];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (int8_t(u >> (8 * e)) < 0) v[4 * q + e] = -v[4 * q + e];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int h = 1; h < V; h <<= 1)
        if (h < b) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (!(e & h)) {
                    const float x0 = v[e], x1 = v[e | h];
                    v[e] = x0 + x1;
                    v[e | h] = x0 - x1;
                }
        }
    for (int h = V; h < b; h <<= 1) {
        const int d = h / V;
        const bool upper = (l & d) != 0;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float p = __shfl_xor(v[e], d);
            v[e] = upper ? p - v[e] : v[e] + p;
        }
    }
    const size_t idx = size_t(t) * n + col;
    if (mode == 0) {
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx);
#pragma unroll
        for (int q = 0; q < V / 4; ++q)
            p[q] = f32x4{v[4 * q] * norm, v[4 * q + 1] * norm, v[4 * q + 2] * norm, v[4 * q + 3] * norm};
    } else {
        u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx);
#pragma unroll
        for (int q = 0; q < V / 8; ++q) {
            u32x4 u;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                u[k] = f2h(v[8 * q + 2 * k] * norm) | (f2h(v[8 * q + 2 * k + 1] * norm) << 16);
            p[q] = u;
        }
    }
}

hipError_t launch_rotate(int T, int n, int b, const void* x, int x_is_f32, const uint16_t* s,
                         const int8_t* sign, void* out, int mode, hipStream_t st) {
    if (mode < 0 || mode > 1 || b < 1 || b > 1024 || (b & (b - 1)) || n % b)
        return hipErrorInvalidValue;
    const int rows = T;
    const float vnorm = float(1.0 / __builtin_sqrt(double(b)));
    auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    if (b <= 1024 && n % (64 * (b <= 512 ? 8 : 16)) == 0 && al16(x) && al16(out) && al16(s) &&
        (reinterpret_cast<uintptr_t>(sign) & 3) == 0) {  // 16-byte accesses
        const int V = b <= 512 ? 8 : 16;
        const int waves = rows * (n / (64 * V));
        const dim3 grid((waves + 3) / 4);
        if (V == 8)
            hipLaunchKernelGGL(k_rotate_v<8>, grid, dim3(256), 0, st, T, rows, n, b, x, x_is_f32, s,
                               sign, out, mode, vnorm);
        else
            hipLaunchKernelGGL(k_rotate_v<16>, grid, dim3(256), 0, st, T, rows, n, b, x, x_is_f32,
                               s, sign, out, mode, vnorm);
        return hipGetLastError();
    }
    const int ne = b <= 64 ? 1 : b / 64;
    const int chunks = (n + 64 * ne - 1) / (64 * ne);
    const int waves = rows * chunks;
    const float norm = float(1.0 / __builtin_sqrt(double(b)));
    const dim3 grid((waves + 3) / 4);
#define VQ_ROT(NE)                                                                        \
    if (ne == NE) {                                                                       \
        hipLaunchKernelGGL(k_rotate<NE>, grid, dim3(256), 0, st, T, rows, n, b, x,        \
                           x_is_f32, s, sign, out, mode, norm);                           \
        return hipGetLastError();                                                         \
    }
    VQ_ROT(1) VQ_ROT(2) VQ_ROT(4) VQ_ROT(8) VQ_ROT(16)
#undef VQ_ROT
    return hipErrorInvalidValue;
}

// Streaming read of a buffer (measurement hook): workgroup b reads its own contiguous share of
// the 16-byte words, 256 threads x 16 bytes per step, and folds them into a XOR the compiler
// cannot drop (the word is stored only when the fold hits one particular value).
__global__ void __launch_bounds__(256) k_stream_read(const u32x4* __restrict__ buf, size_t n16,
                                                     size_t per_wg, uint32_t* sink) {
    const size_t b0 = size_t(blockIdx.x) * per_wg;
    const size_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    size_t i = b0 + threadIdx.x;
    for (; i + 3 * 256 < b1; i += 4 * 256) {
        const u32x4 v0 = __builtin_nontemporal_load(buf + i);
        const u32x4 v1 = __builtin_nontemporal_load(buf + i + 256);
        const u32x4 v2 = __builtin_nontemporal_load(buf + i + 512);
        const u32x4 v3 = __builtin_nontemporal_load(buf + i + 768);
        acc ^= (v0 ^ v1) ^ (v2 ^ v3);
    }
    for (; i < b1; i += 256) acc ^= buf[i];
    const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (r == 0x9E3779B9u) sink[0] = r;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int cus,
                              hipStream_t st) {
    if (!buf || !sink || bytes % 16 || cus < 1) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t grid = size_t(cus) * 8;  // 8 workgroups of 4 waves per CU
    size_t per = (n16 + grid - 1) / grid;
    per = (per + 1023) & ~size_t(1023);  // whole 16 KB steps
    grid = (n16 + per - 1) / per;
    hipLaunchKernelGGL(k_stream_read, dim3(unsigned(grid)), dim3(256), 0, st,
                       static_cast<const u32x4*>(buf), n16, per, sink);
    return hipGetLastError();
}

}  // namespace vqmlp
