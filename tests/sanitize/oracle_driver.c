/* The FP64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the MLP, the scalar-LUT
 * projection, the rotation and the weight decoders on small random inputs (including the
 * argument errors they document), with a round-trip check of the rotation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double orc_f16_to_f64(uint16_t h);
int orc_rotate(int T, int n, int b, const double *u, const int8_t *sign, double *out);
int orc_vq3_weight(int N, int K, const uint8_t *codes, const uint16_t *cb, const uint16_t *sc,
                   double *W);
int orc_vq3_matmul(int T, int N, int K, const uint8_t *codes, const uint16_t *cb,
                   const uint16_t *sc, const double *in, double *out);
int orc_mlp_forward(int T, int H, int I, int bh, int bi, const uint16_t *x, const uint16_t *s,
                    const int8_t *sign_h, const int8_t *sign_i, const uint8_t *c_gate,
                    const uint16_t *cb_gate, const uint16_t *sc_gate, const uint8_t *c_up,
                    const uint16_t *cb_up, const uint16_t *sc_up, const uint8_t *c_down,
                    const uint16_t *cb_down, const uint16_t *sc_down, double *y, double *xt_out,
                    double *g_out, double *v_out, double *a_out, double *at_out);
int orc_lut_weight(int bits, int N, int K, const uint8_t *codes, const uint16_t *lut,
                   const uint16_t *sc, double *W);
int orc_lut_forward(int bits, int N, int K, int T, int b, int rank, const uint16_t *x,
                    const uint16_t *s, const int8_t *sign, const uint8_t *codes,
                    const uint16_t *lut, const uint16_t *sc, const uint16_t *U,
                    const uint16_t *V, double *y, double *xt_out);

static uint32_t st = 777u;
static uint32_t rnd(void) {
    st ^= st << 13;
    st ^= st >> 17;
    st ^= st << 5;
    return st;
}
/* a binary16 of modest magnitude: sign, exponent 10..16, random fraction */
static uint16_t h16(void) { return (uint16_t)(((rnd() & 1) << 15) | ((10 + rnd() % 7) << 10) | (rnd() & 1023)); }

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c); \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main(void) {
    const int T = 3, H = 64, I = 96;
    uint16_t *x = malloc(sizeof(uint16_t) * T * H), *s = malloc(sizeof(uint16_t) * H);
    int8_t *sh = malloc(H), *si = malloc(I);
    uint8_t *cg = malloc((I / 2) * H), *cu = malloc((I / 2) * H), *cd = malloc((H / 2) * I);
    uint16_t *bg = malloc(2 * 64 * 2 * (I / 8)), *bu = malloc(2 * 64 * 2 * (I / 8)),
             *bd = malloc(2 * 64 * 2 * (H / 8));
    uint16_t *sg = malloc(2 * I), *su = malloc(2 * I), *sd = malloc(2 * H);
    for (int i = 0; i < T * H; ++i) x[i] = h16();
    for (int i = 0; i < H; ++i) { s[i] = h16() & 0x7FFF; sh[i] = (rnd() & 1) ? 1 : -1; }
    for (int i = 0; i < I; ++i) { si[i] = (rnd() & 1) ? 1 : -1; sg[i] = su[i] = 0x3C00; }
    for (int i = 0; i < H; ++i) sd[i] = 0x3800;
    for (int i = 0; i < (I / 2) * H; ++i) { cg[i] = rnd() & 63; cu[i] = rnd() & 63; cd[i] = rnd() & 63; }
    for (int i = 0; i < 128 * (I / 8); ++i) { bg[i] = h16() & 0xBFFF; bu[i] = h16() & 0xBFFF; }
    for (int i = 0; i < 128 * (H / 8); ++i) bd[i] = h16() & 0xBFFF;
    double *y = malloc(sizeof(double) * T * H), *xt = malloc(sizeof(double) * T * H);
    double *g = malloc(sizeof(double) * T * I), *v = malloc(sizeof(double) * T * I);
    double *a = malloc(sizeof(double) * T * I), *at = malloc(sizeof(double) * T * I);
    CHECK(orc_mlp_forward(T, H, I, 32, 32, x, s, sh, si, cg, bg, sg, cu, bu, su, cd, bd, sd, y,
                          xt, g, v, a, at) == 0);
    for (int i = 0; i < T * H; ++i) CHECK(isfinite(y[i]));
    CHECK(orc_mlp_forward(T, H, I, 48, 32, x, s, sh, si, cg, bg, sg, cu, bu, su, cd, bd, sd, y,
                          NULL, NULL, NULL, NULL, NULL) == 1);  /* block not a power of two */
    CHECK(orc_mlp_forward(0, H, I, 32, 32, x, s, sh, si, cg, bg, sg, cu, bu, su, cd, bd, sd, y,
                          NULL, NULL, NULL, NULL, NULL) == 0);  /* T = 0 */
    /* rotation round trip: R is symmetric without signs, so R(R u) = u */
    double *u = malloc(sizeof(double) * T * H), *r1 = malloc(sizeof(double) * T * H),
           *r2 = malloc(sizeof(double) * T * H);
    for (int i = 0; i < T * H; ++i) u[i] = orc_f16_to_f64(h16());
    CHECK(orc_rotate(T, H, 64, u, NULL, r1) == 0 && orc_rotate(T, H, 64, r1, NULL, r2) == 0);
    for (int i = 0; i < T * H; ++i) CHECK(fabs(r2[i] - u[i]) <= 1e-12 * (1 + fabs(u[i])));
    CHECK(orc_rotate(T, H, 3, u, NULL, r1) == 1);
    double *W = malloc(sizeof(double) * I * H);
    CHECK(orc_vq3_weight(I, H, cg, bg, sg, W) == 0);
    cg[5] = 64;
    CHECK(orc_vq3_weight(I, H, cg, bg, sg, W) == 1);
    CHECK(orc_vq3_matmul(T, I, H, cu, bu, su, xt, g) == 0);
    /* scalar-LUT projection, 2 and 4 bits, with factors and a rotation */
    const int N = 64, K = 128, R = 16;
    uint8_t *lc = malloc(N * K);
    uint16_t *lt = malloc(2 * 16 * (N / 8)), *ls = malloc(2 * N), *U = malloc(2 * N * R),
             *V = malloc(2 * R * K), *lx = malloc(2 * T * K);
    double *ly = malloc(sizeof(double) * T * N), *lW = malloc(sizeof(double) * N * K);
    for (int i = 0; i < 16 * (N / 8); ++i) lt[i] = h16() & 0xBFFF;
    for (int i = 0; i < N; ++i) ls[i] = 0x3C00;
    for (int i = 0; i < N * R; ++i) U[i] = h16() & 0xBFFF;
    for (int i = 0; i < R * K; ++i) V[i] = h16() & 0xBFFF;
    for (int i = 0; i < T * K; ++i) lx[i] = h16();
    for (int bits = 2; bits <= 4; bits += 2) {
        for (int i = 0; i < N * K; ++i) lc[i] = (uint8_t)(rnd() % (1u << bits));
        CHECK(orc_lut_weight(bits, N, K, lc, lt, ls, lW) == 0);
        CHECK(orc_lut_forward(bits, N, K, T, 64, R, lx, NULL, NULL, lc, lt, ls, U, V, ly, NULL) == 0);
        CHECK(orc_lut_forward(bits, N, K, T, 0, 0, lx, NULL, NULL, lc, lt, ls, NULL, NULL, ly, NULL) == 0);
        lc[7] = (uint8_t)(1u << bits);
        CHECK(orc_lut_weight(bits, N, K, lc, lt, ls, lW) == 1);
    }
    CHECK(orc_lut_forward(3, N, K, T, 0, 0, lx, NULL, NULL, lc, lt, ls, NULL, NULL, ly, NULL) == 1);
    free(x); free(s); free(sh); free(si); free(cg); free(cu); free(cd); free(bg); free(bu); free(bd);
    free(sg); free(su); free(sd); free(y); free(xt); free(g); free(v); free(a); free(at); free(u);
    free(r1); free(r2); free(W); free(lc); free(lt); free(ls); free(U); free(V); free(lx); free(ly);
    free(lW);
    puts("oracle driver: ok");
    return 0;
}
