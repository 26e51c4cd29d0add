/* Host-side exercise of libwq under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (built by tests/test_sanitizers.py; no GPU is touched): the host
 * packer and unpacker on every width and ragged shapes (round trip), the
 * size queries over many shapes, and every argument refusal that the entry
 * points decide before any device work (fake but aligned pointers that are
 * never dereferenced: each call is refused or is an empty no-op). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wq.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)rng_state;
}

#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
            return 1;                                                          \
        }                                                                      \
    } while (0)

int main(void) {
    static const int64_t Ks[] = {128, 256, 384, 640, 1280, 5120};
    for (int b = 2; b <= 8; ++b)
        for (size_t ki = 0; ki < sizeof Ks / sizeof Ks[0]; ++ki)
            for (int64_t N = 1; N <= 7; N += 3) {
                const int64_t K = Ks[ki];
                const int64_t W = wq_packed_words_per_row(K, b);
                CHECK(W == (K * b + 31) / 32);
                uint8_t *c = malloc((size_t)(N * K)), *back = malloc((size_t)(N * K));
                uint32_t *p = malloc((size_t)(N * W) * 4);
                for (int64_t i = 0; i < N * K; ++i) c[i] = (uint8_t)(rnd() & ((1u << b) - 1u));
                CHECK(wq_pack(c, N, K, b, 128, p) == WQ_OK);
                CHECK(wq_unpack(p, N, K, b, back) == WQ_OK);
                CHECK(memcmp(c, back, (size_t)(N * K)) == 0);
                c[N * K - 1] = (uint8_t)(1u << b);  /* out of range: refused, never masked */
                if (b < 8) CHECK(wq_pack(c, N, K, b, 128, p) == WQ_ERR_CODE_RANGE);
                free(c), free(back), free(p);
            }
    CHECK(wq_pack(NULL, 1, 128, 6, 128, NULL) != WQ_OK);
    CHECK(wq_packed_words_per_row(128, 9) == -1);

    for (int b = 0; b <= 9; ++b)
        for (int64_t N = 1; N < 20000; N = N * 3 + 1)
            for (size_t ki = 0; ki < sizeof Ks / sizeof Ks[0]; ++ki) {
                const int64_t K = Ks[ki];
                (void)wq_repacked_bytes(WQ_LAYOUT_TILED, N, K, b, 128);
                (void)wq_repacked_bytes(WQ_LAYOUT_DENSE, N, K, b, (int)K);
                for (int64_t M = 0; M < 10000; M = M * 4 + 1) {
                    (void)wq_workspace_bytes(WQ_OP_GEMM, M, N, K, b, 128);
                    (void)wq_workspace_bytes(WQ_OP_GEMM_A8, M, N, K, b, 128);
                }
                int64_t off[5] = {0, 3, 3, 300, 301};
                (void)wq_grouped_workspace_bytes(off, 4, N, K, b, 128);
            }
    for (int s = -2; s < 20; ++s) CHECK(wq_status_str(s) != NULL);

    /* Refusals decided on the host. */
    void *P = (void *)(uintptr_t)0x100000, *Q = (void *)(uintptr_t)0x100008;
    CHECK(wq_gemm(P, 4, 256, 512, P, WQ_LAYOUT_TILED, NULL, NULL, 9, 128, P, P, 1 << 20, NULL) ==
          WQ_ERR_UNSUPPORTED_BITS);
    CHECK(wq_gemm(Q, 4, 256, 512, P, WQ_LAYOUT_TILED, NULL, NULL, 6, 128, P, P, 1 << 20, NULL) ==
          WQ_ERR_MISALIGNED);
    CHECK(wq_gemm(P, 4, 256, 500, P, WQ_LAYOUT_TILED, NULL, NULL, 6, 128, P, P, 1 << 20, NULL) ==
          WQ_ERR_BAD_GROUP);
    CHECK(wq_gemm(P, 4, 256, 512, P, 5, NULL, NULL, 6, 128, P, P, 1 << 20, NULL) ==
          WQ_ERR_BAD_LAYOUT);
    CHECK(wq_gemm(P, 4, 256, 512, P, WQ_LAYOUT_TILED, NULL, P, 6, 128, P, P, 1 << 20, NULL) ==
          WQ_ERR_ZERO_POINTS);
    CHECK(wq_gemm(P, -1, 256, 512, P, WQ_LAYOUT_TILED, NULL, NULL, 6, 128, P, P, 0, NULL) ==
          WQ_ERR_INVALID_ARG);
    CHECK(wq_gemm(NULL, 0, 256, 512, NULL, WQ_LAYOUT_TILED, NULL, NULL, 6, 128, NULL, NULL, 0,
                  NULL) == WQ_OK);
    CHECK(wq_gemm(P, 4, 64, ((int64_t)1 << 22) + 128, P, WQ_LAYOUT_TILED, NULL, NULL, 6, 128, P,
                  P, 1 << 20, NULL) == WQ_ERR_INVALID_ARG);
    CHECK(wq_gemm_noalloc(P, 4, 256, 512, P, WQ_LAYOUT_TILED, NULL, NULL, 1, 128, P, NULL) ==
          WQ_ERR_UNSUPPORTED_BITS);
    CHECK(wq_gemm_a8(P, 4, 256, 512, P, WQ_LAYOUT_TILED, NULL, NULL, 6, 128, P, 7, P, 1 << 20,
                     NULL) != WQ_OK);
    CHECK(wq_embed(P, P, NULL, 1000, 512, 9, 128, P, 4, P, NULL) == WQ_ERR_UNSUPPORTED_BITS);
    CHECK(wq_embed(NULL, NULL, NULL, 1000, 512, 6, 128, NULL, 0, NULL, NULL) == WQ_OK);
    int64_t bad[3] = {0, 5, 4};
    CHECK(wq_gemm_grouped(P, 4, 256, 512, P, 1 << 20, NULL, bad, 2, 6, 128, P, P, 1 << 20, NULL) ==
          WQ_ERR_INVALID_ARG);
    CHECK(wq_repack(P, P, 64, 512, 6, 128, WQ_LAYOUT_DENSE, P, NULL) == WQ_ERR_BAD_LAYOUT);
    CHECK(wq_unpack_dev(NULL, WQ_LAYOUT_TILED, 64, 512, 6, 128, P, NULL) == WQ_ERR_INVALID_ARG);
    printf("host sanitizer run ok\n");
    return 0;
}
