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

constexpr int kRotRows = 8;

__global__ void __launch_bounds__(256) k_rotate(int T, int n, int b, const void* x, int x_is_f32,
                                                const uint16_t* s, const int8_t* sign, void* out,
                                                int mode, float norm) {
    __shared__ float buf[kRotRows * 1024];
    const int blk = blockIdx.x, t0 = blockIdx.y * kRotRows;
    const int nt = min(kRotRows, T - t0);
    const int cnt = kRotRows * b;
    for (int i = threadIdx.x; i < cnt; i += 256) {
        const int tt = i / b, k = i % b, col = blk * b + k;
        float v = 0.f;
        if (tt < nt) {
            const size_t idx = size_t(t0 + tt) * n + col;
            v = x_is_f32 ? static_cast<const float*>(x)[idx]
                         : h2f(static_cast<const uint16_t*>(x)[idx]);
            if (s) v *= h2f(s[col]);
            if (sign && sign[col] < 0) v = -v;
        }
        buf[i] = v;
    }
    __syncthreads();
    const int half = b / 2;
    for (int h = 1; h < b; h <<= 1) {
        for (int i = threadIdx.x; i < kRotRows * half; i += 256) {
            const int tt = i / half, j = i % half;
            const int lo = (j / h) * 2 * h + (j % h), hi = lo + h;
            const float a = buf[tt * b + lo], c = buf[tt * b + hi];
            buf[tt * b + lo] = a + c;
            buf[tt * b + hi] = a - c;
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < cnt; i += 256) {
        const int tt = i / b, k = i % b, col = blk * b + k;
        const float v = buf[i] * norm;
        if (mode == 0) {
            if (tt < nt) static_cast<float*>(out)[size_t(t0 + tt) * n + col] = v;
        } else if (mode == 1) {
            if (tt < nt) static_cast<uint16_t*>(out)[size_t(t0 + tt) * n + col] = (uint16_t)f2h(v);
        } else if (mode == 3) {
            // skinny operand: 8 rows, rows past T zero
            static_cast<uint16_t*>(out)[size_t(tt) * n + col] = (uint16_t)f2h(v);
        } else {
            // skinny operand: K-step col/16, lane 16*kc + 2*tt + c', dword col%4; component c'
            // of the pair-interleaved product gets the value, the other half stays zero.
            const uint32_t hv = f2h(v);
            const int ks = col / 16, kc = (col % 16) / 4, m = col % 4;
            uint32_t* o = static_cast<uint32_t*>(out);
            const int l0 = 16 * kc + 2 * tt;
            o[(size_t(ks) * 64 + l0) * 4 + m] = hv;
            o[(size_t(ks) * 64 + l0 + 1) * 4 + m] = hv << 16;
        }
    }
}

hipError_t launch_rotate(int T, int n, int b, const void* x, int x_is_f32, const uint16_t* s,
                         const int8_t* sign, void* out, int mode, hipStream_t st) {
    if ((mode == 2 || mode == 3) && T > kSkinnyT) return hipErrorInvalidValue;
    const dim3 grid(n / b, mode >= 2 ? 1 : (T + kRotRows - 1) / kRotRows);
    const float norm = float(1.0 / __builtin_sqrt(double(b)));
    hipLaunchKernelGGL(k_rotate, grid, dim3(256), 0, st, T, n, b, x, x_is_f32, s, sign, out, mode,
                       norm);
    return hipGetLastError();
}

}  // namespace vqmlp
