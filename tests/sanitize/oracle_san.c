/* The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (built by
 * tests/test_sanitizers.py with the oracle's own compiler): every entry point
 * on small random inputs for every width, with ragged shapes. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_words_per_row(int64_t K, int b);
int oracle_pack(const uint8_t *codes, int64_t N, int64_t K, int b, uint32_t *packed);
int oracle_unpack(const uint32_t *packed, int64_t N, int64_t K, int b, uint8_t *codes);
int oracle_wna16(const uint16_t *A, int64_t M, int64_t N, int64_t K, const uint32_t *packed,
                 const uint16_t *scales, const uint8_t *zeros, int b, int group, double *y,
                 double *mag);
int oracle_wna16_points(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                        const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros,
                        int b, int group, const int64_t *m_idx, const int64_t *n_idx, int64_t P,
                        double *y, double *mag);
int oracle_quant_act_i8(const uint16_t *A, int64_t M, int64_t K, int8_t *Aq, float *sa);
int oracle_w4a8(const uint16_t *A, int64_t M, int64_t N, int64_t K, const uint32_t *packed,
                const uint16_t *scales, const uint8_t *zeros, int b, int group, int8_t *Aq,
                float *sa, double *y, double *mag);
int oracle_embed(const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros, int64_t V,
                 int64_t K, int b, int group, const int64_t *ids, int64_t T, uint16_t *out);
int oracle_wna16_grouped(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                         const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros,
                         int b, int group, const int64_t *off, int64_t E, double *y,
                         double *mag);

static uint64_t s = 0x2545F4914F6CDD1Dull;
static uint32_t rnd(void) {
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return (uint32_t)s;
}
static uint16_t rnd_bf16(void) { return (uint16_t)(0x3C00u + (rnd() & 0x07FFu)) ^ (uint16_t)((rnd() & 1u) << 15); }

int main(void) {
    const int64_t M = 3, N = 5, K = 384, G = K / 128;
    for (int b = 2; b <= 8; ++b) {
        const int64_t W = oracle_words_per_row(K, b);
        uint8_t *c = malloc((size_t)(N * K)), *back = malloc((size_t)(N * K));
        uint32_t *p = malloc((size_t)(N * W) * 4 * 2);
        uint16_t *A = malloc((size_t)(M * K) * 2), *sc = malloc((size_t)(N * G) * 2 * 2);
        uint8_t *z = malloc((size_t)(N * G) * 2);
        double *y = malloc((size_t)(M * N) * 8), *mag = malloc((size_t)(M * N) * 8);
        int8_t *Aq = malloc((size_t)(M * K));
        float *sa = malloc((size_t)M * 4);
        uint16_t *emb = malloc((size_t)(4 * K) * 2);
        for (int64_t i = 0; i < N * K; ++i) c[i] = (uint8_t)(rnd() & ((1u << b) - 1u));
        for (int64_t i = 0; i < M * K; ++i) A[i] = rnd_bf16();
        for (int64_t i = 0; i < 2 * N * G; ++i) sc[i] = rnd_bf16(), z[i] = (uint8_t)(rnd() & ((1u << b) - 1u));
        if (oracle_pack(c, N, K, b, p) || oracle_unpack(p, N, K, b, back) ||
            memcmp(c, back, (size_t)(N * K))) {
            fprintf(stderr, "pack round trip failed b=%d\n", b);
            return 1;
        }
        memcpy(p + N * W, p, (size_t)(N * W) * 4);  /* a second expert */
        oracle_wna16(A, M, N, K, p, sc, NULL, b, 128, y, mag);
        oracle_wna16(A, M, N, K, p, sc, z, b, 128, y, mag);
        oracle_wna16(A, M, N, K, p, sc, NULL, b, (int)K, y, NULL);
        int64_t mi[4] = {0, 2, 1, 2}, ni[4] = {4, 0, 3, 1};
        oracle_wna16_points(A, M, N, K, p, sc, NULL, b, 128, mi, ni, 4, y, mag);
        oracle_quant_act_i8(A, M, K, Aq, sa);
        oracle_w4a8(A, M, N, K, p, sc, NULL, b, 128, Aq, sa, y, mag);
        int64_t ids[4] = {0, 4, -1, 7};
        oracle_embed(p, sc, NULL, N, K, b, 128, ids, 4, emb);
        int64_t off[3] = {0, 1, 3};
        oracle_wna16_grouped(A, M, N, K, p, sc, NULL, b, 128, off, 2, y, mag);
        free(c), free(back), free(p), free(A), free(sc), free(z), free(y), free(mag), free(Aq);
        free(sa), free(emb);
    }
    printf("oracle sanitizer run ok\n");
    return 0;
}
