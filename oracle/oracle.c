/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the INT4 group-quantized
 * weight-only linear layer (W4A16) and its greedy-verify epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library: every decode below is written
 * out here from the IEEE-754 and packing definitions.
 *
 * What is computed (sources, all about arXiv 2607.04244 "Quantize the Target,
 * Quantize the Drafter: Efficient Inference with Qwen3.5-4B"):
 *   - the target model runs on an AWQ INT4 grid; distillation keeps its
 *     per-group scales fixed and rounds the trained weights back onto that
 *     grid, so the packed format and the serving path do not change (Pith
 *     review, Referee Report: Summary and Significance; Assumptions & free
 *     parameters, second assumption);
 *   - the drafter's weights are INT4 in groups of 128 (Pith review,
 *     Assumptions & free parameters: the drafter's GPTQ group size);
 *   - verification by the target leaves the output unchanged, so a draft
 *     token survives only while it matches the target's greedy choice (Pith
 *     review, Assumptions & free parameters, first assumption; mlsanity index
 *     page, Abstract).
 * The pages print no formula, layout or worked example.  The readings used
 * (all stated again at each function):
 *   W[n,k] = (q[n,k] - z[n,g]) * s[n,g],  g = floor(k / group)
 *   Y[m,n] = sum_k X[m,k] * W[n,k]
 *   q packed 8 per uint32 along K, nibble j of word w holds k = 8w + j
 *   (low nibble first); z packed 8 per uint32 along N the same way;
 *   s is IEEE binary16, X is bfloat16 (upper half of an IEEE binary32).
 *
 * Everything here is fp64 with naive loops in index order: no blocking, no
 * reordering, no fusion.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- exact decoders ---------------------------------------------------- */

/* bfloat16 is the upper 16 bits of an IEEE-754 binary32: widen and convert. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal: (-1)^s * 2^(e-15) * (1 + f/1024); subnormal: (-1)^s * 2^-14 * f/1024. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* ---- packing (the grid in memory) -------------------------------------- */

/* Pack codes u8[N][K] (values 0..15; higher bits ignored) into
 * qweight u32[N][K/8]: nibble j (bits 4j..4j+3) of word w of row n holds
 * code (n, 8w + j).  Pack zeros u8[N][G] into qzeros u32[N/8][G]: nibble j of
 * word (r, g) holds the zero of row 8r + j, group g.
 * Reading: eight codes per 32-bit word along K, in the plainest order. */
void oracle_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int group,
                 uint32_t *qweight, uint32_t *qzeros)
{
    int G = K / group;
    int KW = K / 8;
    for (int n = 0; n < N; ++n)
        for (int w = 0; w < KW; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j)
                word |= (uint32_t)(codes[(size_t)n * K + 8 * w + j] & 15u) << (4 * j);
            qweight[(size_t)n * KW + w] = word;
        }
    for (int r = 0; r < N / 8; ++r)
        for (int g = 0; g < G; ++g) {
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j)
                word |= (uint32_t)(zeros[(size_t)(8 * r + j) * G + g] & 15u) << (4 * j);
            qzeros[(size_t)r * G + g] = word;
        }
}

/* Inverse of oracle_pack. */
void oracle_unpack(const uint32_t *qweight, const uint32_t *qzeros, int N, int K, int group,
                   uint8_t *codes, uint8_t *zeros)
{
    int G = K / group;
    int KW = K / 8;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            codes[(size_t)n * K + k] =
                (uint8_t)((qweight[(size_t)n * KW + k / 8] >> (4 * (k % 8))) & 15u);
    for (int n = 0; n < N; ++n)
        for (int g = 0; g < G; ++g)
            zeros[(size_t)n * G + g] =
                (uint8_t)((qzeros[(size_t)(n / 8) * G + g] >> (4 * (n % 8))) & 15u);
}

/* ---- the linear layer --------------------------------------------------- */

/* code q[n,k], read straight from the packed word */
static inline int q_at(const uint32_t *qweight, int K, int n, int k)
{
    return (int)((qweight[(size_t)n * (K / 8) + k / 8] >> (4 * (k % 8))) & 15u);
}

/* zero z[n,g], read straight from the packed word */
static inline int z_at(const uint32_t *qzeros, int G, int n, int g)
{
    return (int)((qzeros[(size_t)(n / 8) * G + g] >> (4 * (n % 8))) & 15u);
}

/* Dequantize row n of the weight: W[n,k] = (q - z) * s for the group of k.
 * Exact in fp64: a small integer times an 11-bit significand. */
static void dequant_row(const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                        int n, int K, int group, double *w)
{
    int G = K / group;
    for (int k = 0; k < K; ++k) {
        int g = k / group;
        int q = q_at(qweight, K, n, k);
        int z = z_at(qzeros, G, n, g);
        double s = oracle_f16_to_f64(scales[(size_t)n * G + g]);
        w[k] = (double)(q - z) * s;
    }
}

/* Y[m,n] = sum_{k ascending} X[m,k] * W[n,k], fp64, full output Y f64[M][N].
 * X is bf16 bits [M][K] row-major, scales fp16 bits [N][K/group]. */
void oracle_linear_f64(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales,
                       const uint32_t *qzeros, int M, int N, int K, int group, double *Y)
{
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int n = 0; n < N; ++n) {
            dequant_row(qweight, scales, qzeros, n, K, group, w);
            for (int m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc += oracle_bf16_to_f64(X[(size_t)m * K + k]) * w[k];
                Y[(size_t)m * N + n] = acc;
            }
        }
        free(w);
    }
}

/* GPTQ act-order ("desc_act") variant: column k of the weight belongs to group
 * g_idx[k] instead of floor(k / group), so the groups are sets of columns, not runs
 * (the pages' drafter is GPTQ INT4 with groups of 128: Pith review, Assumptions &
 * free parameters; whether it uses act-order is not said, so both are supported).
 *     Y[m,n] = sum_{k ascending} X[m,k] * (q[n,k] - z[n,g_idx[k]]) * s[n,g_idx[k]]
 * The codes stay in their natural k order in qweight; g_idx i32[K], 0 <= g < K/group.
 * Symmetric GPTQ is the case z = 8 everywhere. */
void oracle_linear_gidx(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales,
                        const uint32_t *qzeros, const int32_t *g_idx, int M, int N, int K, int group,
                        double *Y)
{
    int G = K / group;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int n = 0; n < N; ++n) {
            for (int k = 0; k < K; ++k) {
                int g = g_idx[k];
                w[k] = (double)(q_at(qweight, K, n, k) - z_at(qzeros, G, n, g)) *
                       oracle_f16_to_f64(scales[(size_t)n * G + g]);
            }
            for (int m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc += oracle_bf16_to_f64(X[(size_t)m * K + k]) * w[k];
                Y[(size_t)m * N + n] = acc;
            }
        }
        free(w);
    }
}

/* The same definition evaluated only at the listed (row, col) pairs:
 * out[i] = Y[rows[i], cols[i]].  Used where the full product is too large. */
void oracle_linear_at(const uint16_t *X, const uint32_t *qweight, const uint16_t *scales,
                      const uint32_t *qzeros, int M, int N, int K, int group,
                      const int32_t *rows, const int32_t *cols, int count, double *out)
{
    (void)M;
    (void)N;
    int G = K / group;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < count; ++i) {
        int m = rows[i], n = cols[i];
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
            int g = k / group;
            double w = (double)(q_at(qweight, K, n, k) - z_at(qzeros, G, n, g)) *
                       oracle_f16_to_f64(scales[(size_t)n * G + g]);
            acc += oracle_bf16_to_f64(X[(size_t)m * K + k]) * w;
        }
        out[i] = acc;
    }
}

/* ---- greedy verification ------------------------------------------------ */

/* For each row m of logits Y f64[M][N]:
 *   argmax[m] = the smallest n attaining max_n Y[m,n];
 *   gap[m]    = that maximum minus the largest logit at any other column
 *               (+inf when N == 1).
 * accept_len = the number of leading rows i with argmax[i] == draft[i]
 * (greedy verification keeps draft tokens up to the first one the
 * target would not have chosen). */
void oracle_argmax_accept(const double *Y, int M, int N, const int32_t *draft,
                          int32_t *argmax, double *gap, int32_t *accept_len)
{
    for (int m = 0; m < M; ++m) {
        const double *row = Y + (size_t)m * N;
        int best = 0;
        for (int n = 1; n < N; ++n)
            if (row[n] > row[best])
                best = n;
        double second = -INFINITY;
        for (int n = 0; n < N; ++n)
            if (n != best && row[n] > second)
                second = row[n];
        argmax[m] = best;
        gap[m] = row[best] - second;
    }
    int L = 0;
    while (L < M && argmax[L] == draft[L])
        ++L;
    *accept_len = L;
}

/* ---- re-quantization onto a frozen grid ----------------------------------- */

/* Round a weight matrix back onto the grid, keeping the grid's per-group scales
 * and zero-points (Pith review, Referee Report: Summary and Significance, and
 * Assumptions & free parameters, second assumption: distillation keeps the INT4
 * grid's scales fixed and rounds the trained weights back onto it, so the packed
 * format does not change).  The pages give no formula; the reading is the usual
 * asymmetric one, the inverse of W = (q - z) * s:
 *     q[n,k] = clamp(round(W[n,k] / s[n,g]) + z[n,g], 0, 15),  g = floor(k / group)
 * where round takes the exact quotient to the nearest integer, ties to even, and
 * is applied before z is added (the order matters at exact ties).
 * W u16[N][K] bfloat16 bits, scales u16[N][G] binary16 bits, zeros u8[N][G]
 * (0..15), codes out u8[N][K]. */

/* round(w / s), ties to even, for |w / s| < 32, from exact fp64 arithmetic: w has 8
 * significant bits and s 11, so r * s, w - r * s and 2 (w - r s) - s are exact for
 * the small integers r used here; the fp64 quotient only picks the starting r. */
static double round_quotient(double w, double s)
{
    double r = floor(w / s);
    while (r * s > w) /* make r * s <= w < (r + 1) * s hold exactly */
        r -= 1.0;
    while ((r + 1.0) * s <= w)
        r += 1.0;
    double d = 2.0 * (w - r * s) - s; /* < 0: r is nearer; > 0: r + 1; = 0: a tie */
    if (d > 0.0 || (d == 0.0 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    return r;
}

void oracle_quantize(const uint16_t *W, const uint16_t *scales, const uint8_t *zeros, int N, int K,
                     int group, uint8_t *codes)
{
    int G = K / group;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k) {
            int g = k / group;
            double w = oracle_bf16_to_f64(W[(size_t)n * K + k]);
            double s = oracle_f16_to_f64(scales[(size_t)n * G + g]);
            double z = (double)(zeros[(size_t)n * G + g] & 15u);
            double x = w / s;
            double q;
            if (x != x)            /* NaN weight: the lowest code */
                q = 0.0;
            else if (x >= 32.0)    /* far above the grid (z <= 15): the top code */
                q = 15.0;
            else if (x <= -32.0)   /* far below: the lowest code */
                q = 0.0;
            else
                q = round_quotient(w, s) + z;
            if (q < 0.0)
                q = 0.0;
            if (q > 15.0)
                q = 15.0;
            codes[(size_t)n * K + k] = (uint8_t)q;
        }
}

/* ---- sliding-window attention of a query block (the drafter) ------------- */

/* The drafter attends over a sliding window of the context (Pith review, Assumptions
 * & free parameters: an SWA window of 1024 tokens on the leaderboard, 1024 or 2048 in
 * the window study; inputs of up to 8192 tokens in the pages' Figure 1).  The pages
 * give no kernel or formula; the reading is standard scaled-dot-product attention,
 * causal, over a window, with grouped key/value heads:
 *   queries: the last M tokens of a context of T tokens, query i at position
 *            p_i = T - M + i; head h reads key/value head h / (Hq / Hkv);
 *   keys:    j with p_i - window < j <= p_i (and j >= 0);
 *   O[i,h,:] = sum_j softmax_j(Q[i,h,:] . K[j,kv,:] / sqrt(D)) V[j,kv,:].
 * Layouts: Q [M][Hq][D], K [T][Hkv][D] (token-major), V transposed [Hkv][D][T],
 * all bfloat16 bits; O f64 [M][Hq][D].  fp64 throughout, the softmax shifted by its
 * maximum before the exponentials (exact in real arithmetic). */
void oracle_swa(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, int M, int T, int Hq, int Hkv, int D,
                int window, double *O)
{
    int grp = Hq / Hkv;
    double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(static) collapse(2)
    for (int i = 0; i < M; ++i)
        for (int h = 0; h < Hq; ++h) {
            int kv = h / grp;
            int p = T - M + i;
            int j0 = p - window + 1 > 0 ? p - window + 1 : 0;
            int n = p - j0 + 1;
            double *sc = (double *)malloc(sizeof(double) * (size_t)n);
            double mx = -INFINITY;
            for (int j = j0; j <= p; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += oracle_bf16_to_f64(Q[((size_t)i * Hq + h) * D + d]) *
                           oracle_bf16_to_f64(K[((size_t)j * Hkv + kv) * D + d]);
                sc[j - j0] = dot * scale;
                if (sc[j - j0] > mx)
                    mx = sc[j - j0];
            }
            double sum = 0.0;
            for (int t = 0; t < n; ++t) {
                sc[t] = exp(sc[t] - mx);
                sum += sc[t];
            }
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int j = j0; j <= p; ++j)
                    acc += sc[j - j0] * oracle_bf16_to_f64(Vt[((size_t)kv * D + d) * T + j]);
                O[((size_t)i * Hq + h) * D + d] = acc / sum;
            }
            free(sc);
        }
}

/* The drafter proposes a whole block of tokens at once (mlsanity index page, Builds
 * on: block diffusion for speculative decoding; Pith review, What carries the
 * argument), so its queries may also attend within the block in both directions.
 * Reading of that mode: query i of the block (position p_i = T - M + i) sees every
 * key of the block, T - M <= j < T, and the context keys inside its window,
 * p_i - window < j < T - M (and j >= 0); the rest as oracle_swa. */
void oracle_swa_block(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, int M, int T, int Hq, int Hkv,
                      int D, int window, double *O)
{
    int grp = Hq / Hkv;
    double scale = 1.0 / sqrt((double)D);
    int b0 = T - M; /* first key of the block */
#pragma omp parallel for schedule(static) collapse(2)
    for (int i = 0; i < M; ++i)
        for (int h = 0; h < Hq; ++h) {
            int kv = h / grp;
            int p = b0 + i;
            int c0 = p - window + 1 > 0 ? p - window + 1 : 0; /* first context key in the window */
            if (c0 > b0)
                c0 = b0;
            int j1 = T;      /* one past the last key seen: the whole block */
            int n = j1 - c0; /* the keys c0 .. j1 - 1: the context part, then the block */
            double *sc = (double *)malloc(sizeof(double) * (size_t)n);
            double mx = -INFINITY;
            for (int j = c0; j < j1; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += oracle_bf16_to_f64(Q[((size_t)i * Hq + h) * D + d]) *
                           oracle_bf16_to_f64(K[((size_t)j * Hkv + kv) * D + d]);
                sc[j - c0] = dot * scale;
                if (sc[j - c0] > mx)
                    mx = sc[j - c0];
            }
            double sum = 0.0;
            for (int t = 0; t < n; ++t) {
                sc[t] = exp(sc[t] - mx);
                sum += sc[t];
            }
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int j = c0; j < j1; ++j)
                    acc += sc[j - c0] * oracle_bf16_to_f64(Vt[((size_t)kv * D + d) * T + j]);
                O[((size_t)i * Hq + h) * D + d] = acc / sum;
            }
            free(sc);
        }
}

/* ---- gated MLP activation -------------------------------------------------- */

/* The pages serve a Qwen3.5-4B target (Pith review, Referee Report: Summary) and do
 * not spell out its MLP; the reading is that family's gated form, whose gate and
 * up projections are two of the layer's INT4 linears:
 *   Y[i] = silu(G[i]) * U[i],  silu(g) = g / (1 + exp(-g)) = g * sigmoid(g),
 * with G and U the fp64 results of those projections (oracle_linear_f64). */
void oracle_silu_mul(const double *G, const double *U, long long n, double *Y)
{
    for (long long i = 0; i < n; ++i)
        Y[i] = G[i] / (1.0 + exp(-G[i])) * U[i];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
