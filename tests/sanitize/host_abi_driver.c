/* Host half of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: packing round
 * trips of all three weight formats on several shapes, and every argument error the header
 * documents for calls that need no GPU.  Exits non-zero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vqmlp.h"

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c); \
            return 1;                                                   \
        }                                                               \
    } while (0)

static int vq3_round_trip(int N, int K) {
    size_t n = 0;
    CHECK(vqmlp_packed_bytes(N, K, &n) == VQMLP_OK);
    uint8_t* codes = malloc((size_t)(N / 2) * K);
    uint16_t* cb = malloc((size_t)(N / 8) * 64 * 2 * 2);
    uint16_t* sc = malloc((size_t)N * 2);
    uint8_t* packed = malloc(n);
    uint8_t* codes2 = malloc((size_t)(N / 2) * K);
    uint16_t* cb2 = malloc((size_t)(N / 8) * 64 * 2 * 2);
    uint16_t* sc2 = malloc((size_t)N * 2);
    for (size_t i = 0; i < (size_t)(N / 2) * K; ++i) codes[i] = (uint8_t)(rnd() & 63);
    for (size_t i = 0; i < (size_t)(N / 8) * 128; ++i) cb[i] = (uint16_t)rnd();
    for (int i = 0; i < N; ++i) sc[i] = (uint16_t)rnd();
    CHECK(vqmlp_pack(N, K, codes, cb, sc, packed, n) == VQMLP_OK);
    CHECK(vqmlp_pack(N, K, codes, cb, sc, packed, n - 1) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_unpack(N, K, packed, n, codes2, cb2, sc2) == VQMLP_OK);
    CHECK(memcmp(codes, codes2, (size_t)(N / 2) * K) == 0);
    CHECK(memcmp(cb, cb2, (size_t)(N / 8) * 256) == 0);
    CHECK(memcmp(sc, sc2, (size_t)N * 2) == 0);
    packed[0] ^= 1; /* magic */
    CHECK(vqmlp_unpack(N, K, packed, n, codes2, cb2, sc2) == VQMLP_ERR_INVALID_ARG);
    packed[0] ^= 1;
    codes[(size_t)(N / 2) * K - 1] = 64;
    CHECK(vqmlp_pack(N, K, codes, cb, sc, packed, n) == VQMLP_ERR_INVALID_ARG);
    free(codes); free(cb); free(sc); free(packed); free(codes2); free(cb2); free(sc2);
    return 0;
}

static int lut_round_trip(int bits, int N, int K) {
    size_t n = 0;
    CHECK(vqmlp_lut_packed_bytes(bits, N, K, &n) == VQMLP_OK);
    const int E = 1 << bits;
    uint8_t* codes = malloc((size_t)N * K);
    uint16_t* lut = malloc((size_t)(N / 8) * E * 2);
    uint16_t* sc = malloc((size_t)N * 2);
    uint8_t* packed = malloc(n);
    uint8_t* codes2 = malloc((size_t)N * K);
    uint16_t* lut2 = malloc((size_t)(N / 8) * E * 2);
    uint16_t* sc2 = malloc((size_t)N * 2);
    for (size_t i = 0; i < (size_t)N * K; ++i) codes[i] = (uint8_t)(rnd() % (uint32_t)E);
    for (size_t i = 0; i < (size_t)(N / 8) * E; ++i) lut[i] = (uint16_t)rnd();
    for (int i = 0; i < N; ++i) sc[i] = (uint16_t)rnd();
    CHECK(vqmlp_lut_pack(bits, N, K, codes, lut, sc, packed, n) == VQMLP_OK);
    CHECK(vqmlp_lut_unpack(bits, N, K, packed, n, codes2, lut2, sc2) == VQMLP_OK);
    CHECK(memcmp(codes, codes2, (size_t)N * K) == 0);
    CHECK(memcmp(lut, lut2, (size_t)(N / 8) * E * 2) == 0);
    CHECK(memcmp(sc, sc2, (size_t)N * 2) == 0);
    CHECK(vqmlp_lut_unpack(6 - bits, N, K, packed, n, codes2, lut2, sc2) == VQMLP_ERR_INVALID_ARG);
    codes[0] = (uint8_t)E;
    CHECK(vqmlp_lut_pack(bits, N, K, codes, lut, sc, packed, n) == VQMLP_ERR_INVALID_ARG);
    free(codes); free(lut); free(sc); free(packed); free(codes2); free(lut2); free(sc2);
    return 0;
}

static int vq2_round_trip(int N, int K) {
    size_t n = 0;
    CHECK(vqmlp_vq2_packed_bytes(N, K, &n) == VQMLP_OK);
    uint8_t* codes = malloc((size_t)(N / 2) * K);
    uint16_t* cb = malloc((size_t)(N / 8) * 16 * 2 * 2);
    uint16_t* sc = malloc((size_t)N * 2);
    uint8_t* packed = malloc(n);
    uint8_t* codes2 = malloc((size_t)(N / 2) * K);
    uint16_t* cb2 = malloc((size_t)(N / 8) * 16 * 2 * 2);
    uint16_t* sc2 = malloc((size_t)N * 2);
    for (size_t i = 0; i < (size_t)(N / 2) * K; ++i) codes[i] = (uint8_t)(rnd() & 15);
    for (size_t i = 0; i < (size_t)(N / 8) * 32; ++i) cb[i] = (uint16_t)rnd();
    for (int i = 0; i < N; ++i) sc[i] = (uint16_t)rnd();
    CHECK(vqmlp_vq2_pack(N, K, codes, cb, sc, packed, n) == VQMLP_OK);
    CHECK(vqmlp_vq2_unpack(N, K, packed, n, codes2, cb2, sc2) == VQMLP_OK);
    CHECK(memcmp(codes, codes2, (size_t)(N / 2) * K) == 0);
    CHECK(memcmp(cb, cb2, (size_t)(N / 8) * 64) == 0);
    CHECK(memcmp(sc, sc2, (size_t)N * 2) == 0);
    CHECK(vqmlp_vq2_unpack(N, K, packed, n - 256, codes2, cb2, sc2) == VQMLP_ERR_INVALID_ARG);
    codes[1] = 16;
    CHECK(vqmlp_vq2_pack(N, K, codes, cb, sc, packed, n) == VQMLP_ERR_INVALID_ARG);
    free(codes); free(cb); free(sc); free(packed); free(codes2); free(cb2); free(sc2);
    return 0;
}

int main(void) {
    CHECK(vqmlp_abi_version() == VQMLP_ABI_VERSION);
    const int shapes[][2] = {{32, 64}, {64, 128}, {96, 192}, {256, 704}, {704, 256}};
    for (unsigned i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        if (vq3_round_trip(shapes[i][0], shapes[i][1])) return 1;
    for (int bits = 2; bits <= 4; bits += 2) {
        if (lut_round_trip(bits, 64, 128)) return 1;
        if (lut_round_trip(bits, 128, 1024)) return 1;
    }
    if (vq2_round_trip(32, 32) || vq2_round_trip(96, 160) || vq2_round_trip(256, 512)) return 1;
    /* argument errors that need no device */
    size_t n = 0;
    CHECK(vqmlp_packed_bytes(33, 64, &n) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_packed_bytes(32, 65, &n) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_packed_bytes(32, 64, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_pack(32, 64, NULL, NULL, NULL, NULL, 0) == VQMLP_ERR_INVALID_ARG);
    CHECK(strlen(vqmlp_last_error()) > 0);
    CHECK(vqmlp_lut_packed_bytes(3, 64, 64, &n) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_vq2_packed_bytes(32, 33, &n) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_create(NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_create_vq2(NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_forward(NULL, 1, NULL, NULL, NULL, 0, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_forward_path(NULL, 1, NULL, NULL, NULL, 0, 0, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_forward_noalloc(NULL, 1, NULL, NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_workspace_bytes(NULL, 1, &n) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_workspace_errors(NULL, 0, 0, NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_stream_read(NULL, 0, NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_lut_create(2, 64, 64, NULL, NULL, NULL, 0, NULL, NULL, 0, NULL) != VQMLP_OK);
    CHECK(vqmlp_lut_plan_forward(NULL, 1, NULL, NULL, NULL, 0, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_lut_plan_argmax(NULL, 1, NULL, NULL, NULL, NULL, 0, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_vq2_create(32, 32, NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_vq2_plan_forward(NULL, 1, NULL, NULL, NULL) == VQMLP_ERR_INVALID_ARG);
    CHECK(vqmlp_destroy(NULL) == VQMLP_OK);
    CHECK(vqmlp_lut_destroy(NULL) == VQMLP_OK);
    CHECK(vqmlp_vq2_destroy(NULL) == VQMLP_OK);
    puts("host ABI driver: ok");
    return 0;
}
