/* sanitize_check.c -- test infrastructure: drives every oracle function on small
 * random inputs in exactly-sized heap buffers, for a build with the address and
 * undefined-behaviour sanitizers (a CPU test compiles and runs it).  Also checks a
 * few identities: pack then unpack returns the codes, the sampled linear equals the
 * full one, argmax and accept length stay in range.  Exit status 0 means clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int group, uint32_t *qweight,
                 uint32_t *qzeros);
void oracle_unpack(const uint32_t *qweight, const uint32_t *qzeros, int N, int K, int group, uint8_t *codes,
                   uint8_t *zeros);
void oracle_linear_f64(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                       int M, int N, int K, int group, double *Y);
void oracle_linear_gidx(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                        const int32_t *g_idx, int M, int N, int K, int group, double *Y);
void oracle_linear_at(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                      int M, int N, int K, int group, const int32_t *rows, const int32_t *cols, int count,
                      double *out);
void oracle_argmax_accept(const double *Y, int M, int N, const int32_t *draft, int32_t *argmax, double *gap,
                          int32_t *accept_len);
void oracle_quantize(const uint16_t *W, const uint16_t *scales, const uint8_t *zeros, int N, int K, int group,
                     uint8_t *codes);
void oracle_swa(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, int M, int T, int Hq, int Hkv, int D,
                int window, double *O);
void oracle_swa_block(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, int M, int T, int Hq, int Hkv,
                      int D, int window, double *O);
void oracle_silu_mul(const double *G, const double *U, long long n, double *Y);

static uint32_t rng_state = 12345u;
static uint32_t rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}
/* a bf16 bit pattern of a modest random value */
static uint16_t rbf16(void) { return (uint16_t)(0x3C00u + (rnd() % 0x0600u)) | (uint16_t)((rnd() & 1u) << 15); }

#define CHECK(c)                                                                                             \
    do {                                                                                                     \
        if (!(c)) {                                                                                          \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);                                   \
            return 1;                                                                                        \
        }                                                                                                    \
    } while (0)

int main(void)
{
    const int M = 3, N = 24, K = 384, group = 128, G = K / group;
    uint8_t *codes = malloc((size_t)N * K), *zeros = malloc((size_t)N * G);
    uint8_t *codes2 = malloc((size_t)N * K), *zeros2 = malloc((size_t)N * G);
    uint32_t *qw = malloc((size_t)N * K / 8 * 4), *qz = malloc((size_t)N / 8 * G * 4);
    uint16_t *scales = malloc((size_t)N * G * 2), *X = malloc((size_t)M * K * 2), *W = malloc((size_t)N * K * 2);
    double *Y = malloc((size_t)M * N * 8), *Y2 = malloc((size_t)M * N * 8), *gap = malloc((size_t)M * 8);
    int32_t *g_idx = malloc((size_t)K * 4), *draft = malloc((size_t)M * 4), *am = malloc((size_t)M * 4);
    int32_t *rows = malloc(8 * 4), *cols = malloc(8 * 4), acc = -1;
    double *at = malloc(8 * 8);
    for (int i = 0; i < N * K; ++i)
        codes[i] = (uint8_t)(rnd() & 15u);
    for (int i = 0; i < N * G; ++i) {
        zeros[i] = (uint8_t)(rnd() & 15u);
        scales[i] = (uint16_t)(0x1C00u + rnd() % 0x0800u); /* fp16 in [2^-8, 2^-7) */
    }
    for (int i = 0; i < M * K; ++i)
        X[i] = rbf16();
    oracle_pack(codes, zeros, N, K, group, qw, qz);
    oracle_unpack(qw, qz, N, K, group, codes2, zeros2);
    CHECK(memcmp(codes, codes2, (size_t)N * K) == 0 && memcmp(zeros, zeros2, (size_t)N * G) == 0);
    oracle_linear_f64(X, qw, scales, qz, M, N, K, group, Y);
    for (int k = 0; k < K; ++k)
        g_idx[k] = k / group;
    oracle_linear_gidx(X, qw, scales, qz, g_idx, M, N, K, group, Y2);
    CHECK(memcmp(Y, Y2, (size_t)M * N * 8) == 0);
    for (int i = 0; i < 8; ++i) {
        rows[i] = (int32_t)(rnd() % (uint32_t)M);
        cols[i] = (int32_t)(rnd() % (uint32_t)N);
    }
    oracle_linear_at(X, qw, scales, qz, M, N, K, group, rows, cols, 8, at);
    for (int i = 0; i < 8; ++i)
        CHECK(at[i] == Y[rows[i] * N + cols[i]]);
    for (int i = 0; i < M; ++i)
        draft[i] = (int32_t)(rnd() % (uint32_t)N);
    oracle_argmax_accept(Y, M, N, draft, am, gap, &acc);
    CHECK(acc >= 0 && acc <= M);
    for (int i = 0; i < M; ++i)
        CHECK(am[i] >= 0 && am[i] < N && gap[i] >= 0.0);
    for (int i = 0; i < N * K; ++i)
        W[i] = rbf16();
    oracle_quantize(W, scales, zeros, N, K, group, codes2);
    for (int i = 0; i < N * K; ++i)
        CHECK(codes2[i] <= 15);
    {
        const int Ms = 2, T = 40, Hq = 4, Hkv = 2, D = 128, window = 16;
        uint16_t *Q = malloc((size_t)Ms * Hq * D * 2), *Kc = malloc((size_t)T * Hkv * D * 2);
        uint16_t *Vt = malloc((size_t)Hkv * D * T * 2);
        double *O = malloc((size_t)Ms * Hq * D * 8);
        for (int i = 0; i < Ms * Hq * D; ++i)
            Q[i] = rbf16();
        for (int i = 0; i < T * Hkv * D; ++i) {
            Kc[i] = rbf16();
            Vt[i] = rbf16();
        }
        oracle_swa(Q, Kc, Vt, Ms, T, Hq, Hkv, D, window, O);
        for (int i = 0; i < Ms * Hq * D; ++i)
            CHECK(isfinite(O[i]));
        oracle_swa_block(Q, Kc, Vt, Ms, T, Hq, Hkv, D, window, O);
        for (int i = 0; i < Ms * Hq * D; ++i)
            CHECK(isfinite(O[i]));
        oracle_swa_block(Q, Kc, Vt, Ms, T, Hq, Hkv, D, 1, O);
        free(Q);
        free(Kc);
        free(Vt);
        free(O);
    }
    oracle_silu_mul(Y, Y2, (long long)M * N, Y2);
    free(codes);
    free(zeros);
    free(codes2);
    free(zeros2);
    free(qw);
    free(qz);
    free(scales);
    free(X);
    free(W);
    free(Y);
    free(Y2);
    free(gap);
    free(g_idx);
    free(draft);
    free(am);
    free(rows);
    free(cols);
    free(at);
    printf("oracle sanitize check ok\n");
    return 0;
}
