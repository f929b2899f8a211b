// kernels.hip -- HIP kernels for gfx950 (CDNA4): rotation, dequantisation, the skinny VQ3
// projection for T <= 8 and the tiled matrix-core VQ3 projection for larger T.
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

// ==================================================================== tiled VQ3 projection (T > 8)
//
// D[token][row] = sum_k X[token][k] W[row][k] with v_mfma_f32_16x16x32_f16: A = 16 tokens x 32
// columns of X, B = 32 columns x 16 rows of W decoded into LDS as binary16.  A workgroup owns
// 64 tokens x 64 output rows (of each matrix) and walks K one 64-column tile at a time.

constexpr int kTBM = 64, kTBN = 64, kTBK = 64, kTPad = 8;

template <int NMAT>
__global__ void __launch_bounds__(256) k_tiled(TiledArgs a) {
    __shared__ uint16_t Xs[kTBM][kTBK + kTPad];
    __shared__ uint16_t Ws[NMAT][kTBN][kTBK + kTPad];
    __shared__ uint32_t cbs[NMAT][kTBN / 8][64];
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int N = a.mat[0].N, K = a.mat[0].K, KT = K / kTBK;
    const int nb = blockIdx.x, tb = blockIdx.y;
    const int row0 = nb * kTBN, tok0 = tb * kTBM;
    for (int m = 0; m < NMAT; ++m)
        for (int i = tid; i < (kTBN / 8) * 64; i += 256)
            cbs[m][i / 64][i % 64] = a.mat[m].cb[size_t(row0 / 8) * 64 + i];
    const int wt = (w >> 1) * 32, wr = (w & 1) * 32;  // this wave's 32 tokens x 32 rows
    f32x4 acc[NMAT][2][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
        // X tile: 64 tokens x 64 columns, 16 bytes per thread per pass
        for (int i = tid; i < kTBM * (kTBK / 8); i += 256) {
            const int tt = i / (kTBK / 8), c8 = (i % (kTBK / 8)) * 8;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (tok0 + tt < a.T)
                v = *reinterpret_cast<const u32x4*>(a.xt + size_t(tok0 + tt) * K + kt * kTBK + c8);
            *reinterpret_cast<u32x4*>(&Xs[tt][c8]) = v;
        }
        // W tiles: NMAT x 2 packed tiles x 64 lanes of 16 codes
        for (int task = tid; task < NMAT * 2 * 64; task += 256) {
            const int m = task / 128, pt = (task / 64) & 1, ll = task & 63;
            const int mt = nb * 2 + pt;
            const uint32_t* p = reinterpret_cast<const uint32_t*>(
                a.mat[m].codes + (size_t(mt) * KT + kt) * kTileBytes) + 3 * ll;
            const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
            const int pl = pt * 16 + (ll & 15);
            const uint32_t* tabg = cbs[m][pl >> 2];
            uint16_t* re = Ws[m][2 * pl];
            uint16_t* ro = Ws[m][2 * pl + 1];
            const int cb4 = 4 * (ll >> 4);
#define VQ_DEC(Q)                                                       \
    {                                                                   \
        const uint32_t e = tabg[code_of<Q>(d0, d1, d2)];                \
        const int col = 16 * (Q / 4) + cb4 + (Q % 4);                   \
        re[col] = (uint16_t)(e & 0xFFFFu);                              \
        ro[col] = (uint16_t)(e >> 16);                                  \
    }
            VQ_DEC(0) VQ_DEC(1) VQ_DEC(2) VQ_DEC(3) VQ_DEC(4) VQ_DEC(5) VQ_DEC(6) VQ_DEC(7)
            VQ_DEC(8) VQ_DEC(9) VQ_DEC(10) VQ_DEC(11) VQ_DEC(12) VQ_DEC(13) VQ_DEC(14) VQ_DEC(15)
#undef VQ_DEC
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int kk = ks * 32 + 8 * (l >> 4);
            half8 A[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                A[i] = *reinterpret_cast<const half8*>(&Xs[wt + 16 * i + (l & 15)][kk]);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const half8 Bv = *reinterpret_cast<const half8*>(&Ws[m][wr + 16 * j + (l & 15)][kk]);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], Bv, acc[m][i][j], 0, 0, 0);
                }
        }
    }
    // epilogue: lane l, register r holds D[4*(l/16) + r][l % 16] of each 16x16 sub-tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = tok0 + wt + 16 * i + 4 * (l >> 4) + r;
                const int row = row0 + wr + 16 * j + (l & 15);
                if (tok >= a.T) continue;
                if (NMAT == 2) {
                    const float g = acc[0][i][j][r] * h2f(a.mat[0].sc[row]);
                    const float u = acc[NMAT - 1][i][j][r] * h2f(a.mat[NMAT - 1].sc[row]);
                    float act = g / (1.f + expf(-g)) * u;
                    if (a.sign_i && a.sign_i[row] < 0) act = -act;
                    a.a_out[size_t(tok) * N + row] = act;
                } else {
                    a.y[size_t(tok) * N + row] = (uint16_t)f2h(acc[0][i][j][r] * h2f(a.mat[0].sc[row]));
                }
            }
}

hipError_t launch_tiled(const TiledArgs& a, hipStream_t st) {
    const dim3 grid(a.mat[0].N / kTBN, (a.T + kTBM - 1) / kTBM);
    if (a.nmat == 2)
        hipLaunchKernelGGL(k_tiled<2>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_tiled<1>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace vqmlp
