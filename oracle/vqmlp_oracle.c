/*
 * vqmlp_oracle.c -- plain, slow FP64 CPU reference for the VQ3 quantized-MLP forward and the
 * scalar-LUT projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load this library.  It shares no code, header, table or helper with the HIP library: it
 * has its own binary16 decoding, builds Hadamard signs from the bit-count definition, and
 * decodes every weight from its code on the fly.  Nothing here is blocked, fused or reordered;
 * every sum runs in index order, so results do not depend on the thread count.
 *
 * What is computed, and where it is defined (web pages on "bit_vector_lut"):
 *   - model card "anemll/anemll-forge-qwen3.8-27B", section "Release 0.2: three-bit MLP,
 *     token-mixer rotations, distilled weights": every MLP matrix (gate, up, down) is a three-bit
 *     vector lookup table "2x64": 64 two-component centroids, one six-bit index per pair of output
 *     channels, per-channel scales (format table and first bullet).  Inputs are rotated online
 *     by Hadamard blocks with seeded signs and the weights live in the rotated basis (second
 *     bullet).  Token mixers use two-bit / four-bit lookup tables plus rank-64 FP16 factors
 *     (format table, "Token mixers" row).
 *   - same card, section "Files and runtime compatibility", first bullet: per-channel scaling and
 *     online Hadamard rotations on the MLP and token-mixer inputs.
 *   - "ANEMLL ANE LLM conversion pipeline" (llms-explorer), Facts, item on Forge numerics: the
 *     MLP activation is x*sigmoid(x), written there as 0.5*x*(1+tanh(x/2)).
 *
 * Readings where the pages leave a step open (each is the plainest one the text supports):
 *   - a codebook is shared by each group of 8 output rows (a per-matrix table is the special case
 *     of equal groups); code[p][j] selects the vector (W[2p][j], W[2p+1][j]); component 0 goes to
 *     the even row;
 *   - the row scale multiplies the decoded weight: W[r][j] = cb[r/8][code[r/2][j]][r%2] * sc[r];
 *   - the input scale multiplies: u = x * s;
 *   - a rotation is R = (I_{n/b} (x) H_b / sqrt(b)) * diag(d): the sign is applied first, H_b is
 *     the Sylvester-ordered Hadamard matrix H_b[i][k] = (-1)^popcount(i & k), normalised once;
 *   - MLP: y = W_down * R_I( silu(W_gate * x~) . (W_up * x~) ),  x~ = R_H(x . s), silu(g) =
 *     g / (1 + exp(-g));  there is no second per-channel scale before the down projection;
 *   - scalar-LUT projection: y = W x~ + U (V x~) with x~ = R(x . s) (1024-wide blocks) and
 *     W[n][j] = lut[n/8][code[n][j]] * sc[n].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------- binary16 -> double */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Exponent 0 holds
 * zero and the subnormals m * 2^-24; exponent 31 holds infinities and NaNs. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

void orc_f16_array(size_t n, const uint16_t *h, double *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f64(h[i]);
}

/* ---------------------------------------------------------------- Hadamard rotation */

static int orc_bit_parity(unsigned v)
{
    int p = 0;
    while (v) {
        p ^= 1;
        v &= v - 1;
    }
    return p;
}

/* Entry (i, k) of the unnormalised Sylvester Hadamard matrix: (-1)^popcount(i & k). */
int orc_hadamard_entry(int i, int k)
{
    return orc_bit_parity((unsigned)(i & k)) ? -1 : 1;
}

/* Materialise H_b (b*b int8, row-major). */
void orc_hadamard(int b, int8_t *out)
{
    for (int i = 0; i < b; ++i)
        for (int k = 0; k < b; ++k)
            out[(size_t)i * b + k] = (int8_t)orc_hadamard_entry(i, k);
}

static int orc_is_pow2(int b) { return b > 0 && (b & (b - 1)) == 0; }

/* out[t][B*b + i] = b^-1/2 * sum_k H_b[i][k] * sign[B*b+k] * u[t][B*b + k] for every block B.
 * sign may be NULL (all +1).  The dense definition, O(b) per output; out must not alias u. */
int orc_rotate(int T, int n, int b, const double *u, const int8_t *sign, double *out)
{
    if (!orc_is_pow2(b) || n % b)
        return 1;
    const double norm = 1.0 / sqrt((double)b);
    for (int t = 0; t < T; ++t) {
        const double *ut = u + (size_t)t * n;
        double *ot = out + (size_t)t * n;
        for (int blk = 0; blk < n / b; ++blk) {
            const int base = blk * b;
            for (int i = 0; i < b; ++i) {
                double acc = 0.0;
                for (int k = 0; k < b; ++k) {
                    double v = ut[base + k];
                    if (sign && sign[base + k] < 0)
                        v = -v;
                    acc += orc_hadamard_entry(i, k) < 0 ? -v : v;
                }
                ot[base + i] = acc * norm;
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- activation */

double orc_silu_1(double g) { return g / (1.0 + exp(-g)); }

void orc_silu(size_t n, const double *in, double *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_silu_1(in[i]);
}

/* ---------------------------------------------------------------- VQ3 weights */

/* W[r][j] of a VQ3 matrix with N rows, K columns:
 *   codes [N/2][K] (0..63), cb [N/8][64][2] binary16, sc [N] binary16. */
static double orc_vq3_w(int K, const uint8_t *codes, const uint16_t *cb, const uint16_t *sc,
                        int r, int j)
{
    const int c = codes[(size_t)(r / 2) * K + j];
    const double centroid = orc_f16_to_f64(cb[((size_t)(r / 8) * 64 + c) * 2 + (r % 2)]);
    return centroid * orc_f16_to_f64(sc[r]); /* exact: 11-bit x 11-bit significands */
}

/* Materialise W [N][K] as doubles.  Returns 1 on bad shape or a code above 63. */
int orc_vq3_weight(int N, int K, const uint8_t *codes, const uint16_t *cb, const uint16_t *sc,
                   double *W)
{
    if (N <= 0 || K <= 0 || N % 8)
        return 1;
    for (size_t i = 0; i < (size_t)(N / 2) * K; ++i)
        if (codes[i] > 63)
            return 1;
    for (int r = 0; r < N; ++r)
        for (int j = 0; j < K; ++j)
            W[(size_t)r * K + j] = orc_vq3_w(K, codes, cb, sc, r, j);
    return 0;
}

/* out[t][r] = sum_j W[r][j] * in[t][j], j in index order.  Row r of W is decoded once into a
 * buffer (the definition of W above, entry by entry) and then used for every token: the terms
 * and their order are those of decoding each weight where it is used. */
static int orc_vq3_apply(int T, int N, int K, const uint8_t *codes, const uint16_t *cb,
                         const uint16_t *sc, const double *in, double *out)
{
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        double *wr = malloc(sizeof(double) * (size_t)K);
        if (!wr)
            bad = 1;
#pragma omp for schedule(static)
        for (int r = 0; r < N; ++r) {
            if (!wr)
                continue;
            for (int j = 0; j < K; ++j)
                wr[j] = orc_vq3_w(K, codes, cb, sc, r, j);
            for (int t = 0; t < T; ++t) {
                const double *it = in + (size_t)t * K;
                double acc = 0.0;
                for (int j = 0; j < K; ++j)
                    acc += wr[j] * it[j];
                out[(size_t)t * N + r] = acc;
            }
        }
        free(wr);
    }
    return bad;
}

/* Public form of the product above (used by the dequantisation pins). */
int orc_vq3_matmul(int T, int N, int K, const uint8_t *codes, const uint16_t *cb,
                   const uint16_t *sc, const double *in, double *out)
{
    if (N <= 0 || K <= 0 || N % 8 || T < 0)
        return 1;
    return orc_vq3_apply(T, N, K, codes, cb, sc, in, out);
}

/* ---------------------------------------------------------------- the MLP forward */

/* x [T][H] binary16, s [H] binary16, sign_h [H] / sign_i [I] (+-1, NULL = +1).
 * Gate/up: N=I, K=H.  Down: N=H, K=I.  y [T][H] doubles.  Optional outputs (may be NULL):
 * xt [T][H] rotated input, g and v [T][I] projections, a [T][I] gated product, at [T][I] its
 * rotation.  Returns 0, or 1 on a bad shape or block size. */
int orc_mlp_forward(int T, int H, int I, int bh, int bi,
                    const uint16_t *x, const uint16_t *s, const int8_t *sign_h, const int8_t *sign_i,
                    const uint8_t *c_gate, const uint16_t *cb_gate, const uint16_t *sc_gate,
                    const uint8_t *c_up, const uint16_t *cb_up, const uint16_t *sc_up,
                    const uint8_t *c_down, const uint16_t *cb_down, const uint16_t *sc_down,
                    double *y, double *xt_out, double *g_out, double *v_out, double *a_out,
                    double *at_out)
{
    if (T < 0 || H <= 0 || I <= 0 || H % 8 || I % 8)
        return 1;
    if (!orc_is_pow2(bh) || !orc_is_pow2(bi) || H % bh || I % bi)
        return 1;
    if (T == 0)
        return 0;
    double *u = malloc(sizeof(double) * (size_t)T * H);
    double *xt = malloc(sizeof(double) * (size_t)T * H);
    double *g = malloc(sizeof(double) * (size_t)T * I);
    double *v = malloc(sizeof(double) * (size_t)T * I);
    double *a = malloc(sizeof(double) * (size_t)T * I);
    double *at = malloc(sizeof(double) * (size_t)T * I);
    int rc = 1;
    if (!u || !xt || !g || !v || !a || !at)
        goto done;

    /* 1. per-channel scale (the sign is part of the rotation) */
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < H; ++j)
            u[(size_t)t * H + j] = orc_f16_to_f64(x[(size_t)t * H + j]) * orc_f16_to_f64(s[j]);
    /* 2. rotation of the input */
    if (orc_rotate(T, H, bh, u, sign_h, xt))
        goto done;
    /* 3. gate and up projections */
    if (orc_vq3_apply(T, I, H, c_gate, cb_gate, sc_gate, xt, g) ||
        orc_vq3_apply(T, I, H, c_up, cb_up, sc_up, xt, v))
        goto done;
    /* 4. gated product */
    for (size_t i = 0; i < (size_t)T * I; ++i)
        a[i] = orc_silu_1(g[i]) * v[i];
    /* 5. rotation of the down projection's input (its signs come first, inside orc_rotate) */
    if (orc_rotate(T, I, bi, a, sign_i, at))
        goto done;
    /* 6. down projection */
    if (orc_vq3_apply(T, H, I, c_down, cb_down, sc_down, at, y))
        goto done;

    if (xt_out)
        for (size_t i = 0; i < (size_t)T * H; ++i) xt_out[i] = xt[i];
    if (g_out)
        for (size_t i = 0; i < (size_t)T * I; ++i) g_out[i] = g[i];
    if (v_out)
        for (size_t i = 0; i < (size_t)T * I; ++i) v_out[i] = v[i];
    if (a_out)
        for (size_t i = 0; i < (size_t)T * I; ++i) a_out[i] = a[i];
    if (at_out)
        for (size_t i = 0; i < (size_t)T * I; ++i) at_out[i] = at[i];
    rc = 0;
done:
    free(u);
    free(xt);
    free(g);
    free(v);
    free(a);
    free(at);
    return rc;
}

/* ---------------------------------------------------------------- scalar-LUT projection */

/* W[n][j] = lut[n/8][code[n][j]] * sc[n]; codes [N][K] < 2^bits; lut [N/8][2^bits]. */
static double orc_lut_w(int bits, int K, const uint8_t *codes, const uint16_t *lut,
                        const uint16_t *sc, int n, int j)
{
    const int c = codes[(size_t)n * K + j];
    return orc_f16_to_f64(lut[(size_t)(n / 8) * (1 << bits) + c]) * orc_f16_to_f64(sc[n]);
}

int orc_lut_weight(int bits, int N, int K, const uint8_t *codes, const uint16_t *lut,
                   const uint16_t *sc, double *W)
{
    if ((bits != 2 && bits != 4) || N <= 0 || K <= 0 || N % 8)
        return 1;
    for (size_t i = 0; i < (size_t)N * K; ++i)
        if (codes[i] >= (1u << bits))
            return 1;
    for (int n = 0; n < N; ++n)
        for (int j = 0; j < K; ++j)
            W[(size_t)n * K + j] = orc_lut_w(bits, K, codes, lut, sc, n, j);
    return 0;
}

/* y [T][N] = W x~ + U (V x~), x~ = rotation (block b, signs) of x . s.  s, sign may be NULL;
 * b == 0 means no rotation; rank == 0 (or U/V NULL) means no factors.  xt_out optional. */
int orc_lut_forward(int bits, int N, int K, int T, int b, int rank,
                    const uint16_t *x, const uint16_t *s, const int8_t *sign,
                    const uint8_t *codes, const uint16_t *lut, const uint16_t *sc,
                    const uint16_t *U, const uint16_t *V, double *y, double *xt_out)
{
    if ((bits != 2 && bits != 4) || N <= 0 || K <= 0 || N % 8 || T < 0 || rank < 0)
        return 1;
    if (b && (!orc_is_pow2(b) || K % b))
        return 1;
    if (T == 0)
        return 0;
    double *u = malloc(sizeof(double) * (size_t)T * K);
    double *xt = malloc(sizeof(double) * (size_t)T * K);
    double *z = malloc(sizeof(double) * ((size_t)T * (rank ? rank : 1)));
    int rc = 1;
    if (!u || !xt || !z)
        goto done;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j) {
            double v = orc_f16_to_f64(x[(size_t)t * K + j]);
            if (s)
                v *= orc_f16_to_f64(s[j]);
            u[(size_t)t * K + j] = v;
        }
    if (b) {
        if (orc_rotate(T, K, b, u, sign, xt))
            goto done;
    } else {
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < K; ++j) {
                double v = u[(size_t)t * K + j];
                xt[(size_t)t * K + j] = (sign && sign[j] < 0) ? -v : v;
            }
    }
    const int use_lr = rank > 0 && U && V;
    if (use_lr)
        for (int t = 0; t < T; ++t)
            for (int q = 0; q < rank; ++q) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j)
                    acc += orc_f16_to_f64(V[(size_t)q * K + j]) * xt[(size_t)t * K + j];
                z[(size_t)t * rank + q] = acc;
            }
    /* row n of W decoded once, then used for every token (same terms, same order) */
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        double *wr = malloc(sizeof(double) * (size_t)K);
        if (!wr)
            bad = 1;
#pragma omp for schedule(static)
        for (int n = 0; n < N; ++n) {
            if (!wr)
                continue;
            for (int j = 0; j < K; ++j)
                wr[j] = orc_lut_w(bits, K, codes, lut, sc, n, j);
            for (int t = 0; t < T; ++t) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j)
                    acc += wr[j] * xt[(size_t)t * K + j];
                if (use_lr) {
                    double lr = 0.0;
                    for (int q = 0; q < rank; ++q)
                        lr += orc_f16_to_f64(U[(size_t)n * rank + q]) * z[(size_t)t * rank + q];
                    acc += lr;
                }
                y[(size_t)t * N + n] = acc;
            }
        }
        free(wr);
    }
    if (bad)
        goto done;
    if (xt_out)
        for (size_t i = 0; i < (size_t)T * K; ++i) xt_out[i] = xt[i];
    rc = 0;
done:
    free(u);
    free(xt);
    free(z);
    return rc;
}

/* Thread count of the OpenMP loops (for timing the oracle on one core and on all of them). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
