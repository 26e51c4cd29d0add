/*
 * oracle.c -- plain CPU oracle for the b-bit weight-only quantized linear
 * layer (WNA16) and its int8-activation variant (W4A8).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the GPU library never
 * does, and the two share no source, header or table.  Everything here is
 * written for obviousness, not speed: the bitstream is read and written one
 * bit at a time, arithmetic is fp64 (the int8 activation step is fp32
 * because that step is defined in fp32, see below), loops are naive.
 *
 * Definitions followed (page title, then section):
 *
 *  - Packing.  "Qwen3.8-27B-INT6-Mixed-AutoRound" model card, Findings: the
 *    compressed-tensors pack-quantized layout is dense along in_features,
 *    ceil(in_features * bits / 32) 32-bit words per output row, so codes of
 *    5/6/7 bits straddle word boundaries, while the older per-word formula
 *    (32 // bits codes per word, no straddling) only agrees for widths that
 *    divide 32.  Reading taken here: stream bit i of a row is bit (i % 32) of
 *    word i / 32 (little-endian words, so also bit i % 8 of byte i / 8); code
 *    k occupies stream bits [k*b, k*b + b), least significant bit first;
 *    each row is its own stream, zero-padded to a whole word.
 *
 *  - Symmetric groups.  Same model card, Findings: above four bits there is
 *    no zero point, so every group is symmetric.  Reading: the signed value
 *    of an unsigned code c is q = c - 2^(b-1); one scale per group of 128
 *    consecutive input features (the G128 grouping of "vLLM Quantization",
 *    Qwen3-8B demo); negative scales are legal (club-3090 discussion #733,
 *    "Under the hood").
 *
 *  - The layer's result.  "vLLM Can Run INT5-7", section 2: variants are
 *    compared by dequantizing the weights and running the same F.linear, so
 *    y = A . dequant(W)^T with W of shape [out_features N, in_features K],
 *    no bias.  Here dequant is done in fp64 and the sum is exact-as-fp64.
 *
 *  - Zero points and per-channel scales.  Same model card, Findings: the
 *    asymmetric (zero-point) form exists for 4 and 8 bits only; "vLLM
 *    Quantization" (online shorthands) lists INT8 weights with one scale
 *    per channel.  Reading taken: a zero point is an unsigned integer z per
 *    (row, 128 codes) with the code's range, q = c - z replacing c - 2^(b-1)
 *    (zeros == NULL is the symmetric case), whatever the scale grouping; a
 *    per-channel scale is the group size K (one scale per row).
 *
 *  - Grouped (mixture-of-experts) layer.  Same model card, Findings: the
 *    native checkpoint format has a fused MoE path and the dense layout
 *    does not.  Reading taken: E experts, each a layer of the shape above
 *    with its own codes, scales (and zero points); the rows of A are sorted
 *    by expert, expert e owning rows [off[e], off[e+1]); each row goes
 *    through its expert's layer.
 *
 *  - Quantized embedding gather.  Same model card, Findings: an embedding
 *    table in this dense layout needs a gather that reads the dense rows
 *    (the one it names assumes codes never straddle a word); "vLLM Can Run
 *    INT5-7", section 3: the vocabulary tables (248,320 x 5,120) are worth
 *    quantizing.  Reading taken: row t of the result is row ids[t] of the
 *    table dequantized as above and rounded once to bf16 (nearest, ties to
 *    even); an id outside the table gives a row of zeros (the rows of a
 *    vocabulary shard that belong to other shards).
 *
 *  - W4A8.  club-3090 discussion #733, "Under the hood": activations are
 *    quantized per token to int8 at run time, int4 weights are widened to
 *    int8 without loss, the product runs on int8 units ("Which slugs": the
 *    widening must be lossless, which rules out float formats; integer codes
 *    of any b <= 8 widen losslessly as c - 2^(b-1) in [-128, 127], so the
 *    same definition is kept for every b, b = 4 being W4A8).  Reading taken
 *    (the page gives no formula): s_a = amax_k |a| / 127 in fp32 with IEEE
 *    division, Aq = clamp(rint(a / s_a), -127, 127) with ties to even, a
 *    zero row gives s_a = 0 and Aq = 0; per group of 128 the int products
 *    are summed exactly, then scaled by the group scale, summed over groups
 *    and scaled by s_a.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI 1

int oracle_abi(void) { return ORACLE_ABI; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* 1 on a little-endian host; the byte view of the u32 words relies on it. */
int oracle_little_endian(void) {
    const uint32_t probe = 1u;
    return *(const uint8_t *)&probe == 1u;
}

int64_t oracle_words_per_row(int64_t K, int b) {
    return (K * (int64_t)b + 31) / 32;
}

/* bf16 bit pattern -> double, exactly (bf16 is the top half of an fp32). */
static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Read stream bit i of a row given as bytes. */
static unsigned get_bit(const uint8_t *row, int64_t i) {
    return (row[i >> 3] >> (i & 7)) & 1u;
}

static void set_bit(uint8_t *row, int64_t i) {
    row[i >> 3] = (uint8_t)(row[i >> 3] | (1u << (i & 7)));
}

/* Code k of a row: stream bits [k*b, k*b+b), LSB first. */
static unsigned read_code(const uint8_t *row, int64_t k, int b) {
    unsigned c = 0;
    for (int j = 0; j < b; ++j)
        c |= get_bit(row, k * b + j) << j;
    return c;
}

/* codes uint8 [N,K] -> packed u32 [N, words_per_row].  Returns 0, or -1 when
 * a code does not fit in b bits, or the host is not little-endian. */
int oracle_pack(const uint8_t *codes, int64_t N, int64_t K, int b, uint32_t *packed) {
    if (!oracle_little_endian()) return -1;
    const int64_t W = oracle_words_per_row(K, b);
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *row = (uint8_t *)(packed + n * W);
        memset(row, 0, (size_t)W * 4);
        for (int64_t k = 0; k < K; ++k) {
            unsigned c = codes[n * K + k];
            if (c >> b) return -1;
            for (int j = 0; j < b; ++j)
                if ((c >> j) & 1u) set_bit(row, k * b + j);
        }
    }
    return 0;
}

/* packed u32 [N, words_per_row] -> codes uint8 [N,K]. */
int oracle_unpack(const uint32_t *packed, int64_t N, int64_t K, int b, uint8_t *codes) {
    if (!oracle_little_endian()) return -1;
    const int64_t W = oracle_words_per_row(K, b);
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *row = (const uint8_t *)(packed + n * W);
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)read_code(row, k, b);
    }
    return 0;
}

/* Zero point of row n at code k: zeros[n, k/128] ([N, K/128]), or 2^(b-1)
 * when zeros is NULL. */
static int zero_point(const uint8_t *zeros, int64_t n, int64_t K, int64_t k, int b) {
    return zeros ? (int)zeros[n * (K / 128) + k / 128] : 1 << (b - 1);
}

/* Row n dequantized to fp64: w[k] = s[n, k/group] * (c[n,k] - z[n, k/128]). */
static void dequant_row(const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros,
                        int64_t n, int64_t K, int b, int group, double *w) {
    const int64_t W = oracle_words_per_row(K, b);
    const int64_t G = K / group;
    const uint8_t *row = (const uint8_t *)(packed + n * W);
    for (int64_t k = 0; k < K; ++k) {
        const int q = (int)read_code(row, k, b) - zero_point(zeros, n, K, k, b);
        w[k] = bf16_to_double(scales[n * G + k / group]) * (double)q;
    }
}

/* Nearest bf16 to x, ties to even, as a bit pattern.  Written out from the
 * definition: an 8-significant-bit value whose exponent is that of x (the
 * smallest quantum is 2^-133, bf16's subnormal step), the integer multiple of
 * the quantum chosen by nearbyint() in the default round-to-nearest-even
 * mode, infinity past the largest finite bf16 (2 - 2^-7) * 2^127. */
uint16_t oracle_bf16_rne(double x) {
    if (isnan(x)) return 0x7FC0;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int q = e - 8;
    if (q < -133) q = -133;
    const double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r > ldexp(2.0 - ldexp(1.0, -7), 127)) return (uint16_t)(sign | 0x7F80);
    const float f = (float)r; /* r is a bf16 value, so exact in fp32 */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* Quantized embedding gather: out[t, k] = bf16 of row ids[t] of the
 * dequantized table (zeros for ids outside [0, V)).  packed is the dense
 * [V, ceil(K*b/32)] table, scales bf16 [V, K/group], out bf16 bits [T, K]. */
int oracle_embed(const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros, int64_t V,
                 int64_t K, int b, int group, const int64_t *ids, int64_t T, uint16_t *out) {
    if (!oracle_little_endian() || b < 2 || b > 8 || group <= 0 || K % group) return -1;
    double *w = (double *)malloc((size_t)K * sizeof(double));
    if (!w) return -2;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t id = ids[t];
        if (id < 0 || id >= V) {
            for (int64_t k = 0; k < K; ++k) out[t * K + k] = 0;
            continue;
        }
        dequant_row(packed, scales, zeros, id, K, b, group, w);
        for (int64_t k = 0; k < K; ++k) out[t * K + k] = oracle_bf16_rne(w[k]);
    }
    free(w);
    return 0;
}

/* y[m,n] = sum_k A[m,k] * w[n,k] and mag[m,n] = sum_k |A[m,k] * w[n,k]|,
 * both fp64, outputs [M, N] row-major.  mag may be NULL. */
int oracle_wna16(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                 const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros, int b,
                 int group, double *y, double *mag) {
    if (!oracle_little_endian() || b < 1 || b > 8 || group <= 0 || K % group) return -1;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)K * sizeof(double));
        if (!w) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            if (!w) continue;
            dequant_row(packed, scales, zeros, n, K, b, group, w);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0, acc_abs = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double t = bf16_to_double(A[m * K + k]) * w[k];
                    acc += t;
                    acc_abs += fabs(t);
                }
                y[m * N + n] = acc;
                if (mag) mag[m * N + n] = acc_abs;
            }
        }
        free(w);
    }
    return err;
}

/* The same sums at P chosen output positions (m_idx[p], n_idx[p]). */
int oracle_wna16_points(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                        const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros,
                        int b, int group,
                        const int64_t *m_idx, const int64_t *n_idx, int64_t P,
                        double *y, double *mag) {
    if (!oracle_little_endian() || b < 1 || b > 8 || group <= 0 || K % group) return -1;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t p = 0; p < P; ++p) {
            const int64_t m = m_idx[p], n = n_idx[p];
            if (!w || m < 0 || m >= M || n < 0 || n >= N) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            dequant_row(packed, scales, zeros, n, K, b, group, w);
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double t = bf16_to_double(A[m * K + k]) * w[k];
                acc += t;
                acc_abs += fabs(t);
            }
            y[p] = acc;
            if (mag) mag[p] = acc_abs;
        }
        free(w);
    }
    return err;
}

/* Per-token int8 activation quantization, fp32:
 * s_a[m] = max_k |A[m,k]| / 127;  Aq = clamp(rint(A / s_a), -127, 127);
 * a row of zeros gives s_a = 0 and Aq = 0. */
int oracle_quant_act_i8(const uint16_t *A, int64_t M, int64_t K, int8_t *Aq, float *sa) {
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf(bf16_to_float(A[m * K + k]));
            if (v > amax) amax = v;
        }
        const float s = amax / 127.0f;
        sa[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            int8_t qv = 0;
            if (amax > 0.0f) {
                float r = rintf(bf16_to_float(A[m * K + k]) / s);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                qv = (int8_t)r;
            }
            Aq[m * K + k] = qv;
        }
    }
    return 0;
}

/* One int8-activation output from an already quantized activation row:
 * y = s_a * sum_g s[n,g] * (sum_{k in g} Aq[k] * (c[n,k] - z[n,k/128])),
 * with the inner sums exact in int64 (they must fit int32) and the rest fp64.
 * z_row is row n of the zero points, [K/128] (NULL: 2^(b-1)). */
static int w4a8_dot(const int8_t *aq_row, float sa, const uint8_t *codes_row, int b,
                    const uint16_t *s_row, const uint8_t *z_row, int64_t K, int group,
                    double *y, double *mag) {
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t g = 0; g < K / group; ++g) {
        int64_t ig = 0;
        for (int64_t k = g * group; k < (g + 1) * group; ++k) {
            const int64_t zero = z_row ? (int64_t)z_row[k / 128] : (int64_t)1 << (b - 1);
            ig += (int64_t)aq_row[k] * ((int64_t)codes_row[k] - zero);
        }
        if (ig > INT32_MAX || ig < INT32_MIN) return -3;
        const double t = bf16_to_double(s_row[g]) * (double)ig;
        acc += t;
        acc_abs += fabs(t);
    }
    *y = (double)sa * acc;
    if (mag) *mag = fabs((double)sa) * acc_abs;
    return 0;
}

static void unpack_row(const uint32_t *packed, int64_t n, int64_t K, int b, uint8_t *out) {
    const uint8_t *row = (const uint8_t *)(packed + n * oracle_words_per_row(K, b));
    for (int64_t k = 0; k < K; ++k) out[k] = (uint8_t)read_code(row, k, b);
}

/* Full int8-activation layer on b-bit codes (b = 4: W4A8).  Aq [M,K] and
 * sa [M] are written too (caller provides them).  y, mag: [M, N] fp64. */
int oracle_w4a8(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros, int b,
                int group,
                int8_t *Aq, float *sa, double *y, double *mag) {
    if (!oracle_little_endian() || b < 2 || b > 8 || group <= 0 || K % group) return -1;
    oracle_quant_act_i8(A, M, K, Aq, sa);
    const int64_t G = K / group;
    int err = 0;
#pragma omp parallel
    {
        uint8_t *c = (uint8_t *)malloc((size_t)K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            if (!c) {
#pragma omp atomic write
                err = -2;
                continue;
            }
            unpack_row(packed, n, K, b, c);
            for (int64_t m = 0; m < M; ++m) {
                int r = w4a8_dot(Aq + m * K, sa[m], c, b, scales + n * G,
                                 zeros ? zeros + n * (K / 128) : NULL, K, group,
                                 &y[m * N + n], mag ? &mag[m * N + n] : NULL);
                if (r) {
#pragma omp atomic write
                    err = r;
                }
            }
        }
        free(c);
    }
    return err;
}

/* The int8-activation layer at P chosen output positions; Aq/sa must come
 * from oracle_quant_act_i8 on the same A. */
int oracle_w4a8_points(const int8_t *Aq, const float *sa, int64_t M, int64_t N, int64_t K,
                       const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros,
                       int b, int group,
                       const int64_t *m_idx, const int64_t *n_idx, int64_t P,
                       double *y, double *mag) {
    if (!oracle_little_endian() || b < 2 || b > 8 || group <= 0 || K % group) return -1;
    const int64_t G = K / group;
    int err = 0;
#pragma omp parallel
    {
        uint8_t *c = (uint8_t *)malloc((size_t)K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t p = 0; p < P; ++p) {
            const int64_t m = m_idx[p], n = n_idx[p];
            if (!c || m < 0 || m >= M || n < 0 || n >= N) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            unpack_row(packed, n, K, b, c);
            int r = w4a8_dot(Aq + m * K, sa[m], c, b, scales + n * G,
                             zeros ? zeros + n * (K / 128) : NULL, K, group, &y[p], mag ? &mag[p] : NULL);
            if (r) {
#pragma omp atomic write
                err = r;
            }
        }
        free(c);
    }
    return err;
}

/* Grouped layer: for expert e, rows [off[e], off[e+1]) of A through expert
 * e's layer (packed rows e*N .. e*N+N-1 of the stacked [E*N, W] codes, its
 * scales [E*N, K/group] and zero points [E*N, K/128] rows likewise).
 * off[0] = 0, off[E] = M, nondecreasing.  y, mag: [M, N]. */
int oracle_wna16_grouped(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                         const uint32_t *packed, const uint16_t *scales, const uint8_t *zeros,
                         int b, int group, const int64_t *off, int64_t E, double *y, double *mag) {
    if (off[0] != 0 || off[E] != M || group <= 0 || K % group) return -1;
    const int64_t W = oracle_words_per_row(K, b);
    for (int64_t e = 0; e < E; ++e) {
        const int64_t m0 = off[e], me = off[e + 1] - off[e];
        if (me < 0) return -1;
        if (me == 0) continue;
        const int r = oracle_wna16(A + m0 * K, me, N, K, packed + e * N * W,
                                   scales + e * N * (K / group),
                                   zeros ? zeros + e * N * (K / 128) : NULL, b, group,
                                   y + m0 * N, mag ? mag + m0 * N : NULL);
        if (r) return r;
    }
    return 0;
}
