/* Drives every entry point of the CPU oracle (oracle/oracle.c) over edge-case
 * shapes and values, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py compiles both files
 * together).  The checks here are invariants that hold whatever the values;
 * the numerical pins live in the Python tests.  Exit status 0: every call
 * returned as expected and the sanitizers found nothing. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_double(uint16_t b);
double oracle_e2m1_decode(uint8_t nibble);
uint8_t oracle_e2m1_round(double r);
double oracle_e4m3_decode(uint8_t b);
uint8_t oracle_e4m3_round(double v);
float oracle_alpha_from_amax(float amax);
int oracle_compute_alpha(const uint16_t *A, int64_t R, int64_t K, int64_t lda, const int32_t *idx, int32_t k,
                         float *alpha);
int oracle_alpha_from_absmax(const float *absmax, int64_t K, const int32_t *idx, int32_t k, float *alpha);
int oracle_quantize_nvfp4(const uint16_t *A, int64_t R, int64_t K, int64_t lda, const int32_t *idx, int32_t k,
                          float alpha, uint8_t *codes, uint8_t *scales, uint16_t *side);
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float alpha, int64_t R, int64_t K, double *out);
int oracle_splice_gemm(const uint8_t *Xq, const uint8_t *Xs, float alpha_x, const uint16_t *X_S,
                       const uint8_t *Wq, const uint8_t *Ws, float alpha_w, const uint16_t *W_S,
                       int64_t M, int64_t N, int64_t K, int32_t k, float *Y, int64_t ldy);
int oracle_nvfp4_gemm(const uint8_t *Xq, const uint8_t *Xs, float alpha_x, const uint8_t *Wq, const uint8_t *Ws,
                      float alpha_w, int64_t M, int64_t N, int64_t K, float *Y, int64_t ldy);
int oracle_bf16_gemm(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N, int64_t K, int64_t ldx,
                     int64_t ldw, float *Y, double *Y64);
int oracle_stats(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int64_t *count, double *mean, double *m2,
                 float *absmax);
int oracle_select_topk(const double *m2, int64_t K, int32_t k, int32_t *idx);
int oracle_second_moments(const double *mean, const double *m2, int64_t n, int64_t K, double *out);
int oracle_select_channels(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int32_t k, int64_t *count,
                           double *mean, double *m2, float *absmax, int32_t *idx, float *alpha_x);
int oracle_tim_filter(const float *logp, int64_t B, int64_t ldl, const int32_t *len, float log_tau, int64_t k1_num,
                      int64_t k1_den, int64_t k2, uint8_t *keep, int32_t *g1, int32_t *g2, float *adv,
                      int64_t adv_cols, int64_t lda);

static int failures = 0;
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            failures++;                                                        \
        }                                                                      \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)    /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* finite bf16 patterns of every kind: zeros of both signs, subnormals,
 * normals over the whole range, the largest finite value */
static uint16_t any_bf16(void)
{
    const uint64_t r = next_u64();
    switch (r % 8) {
    case 0: return (uint16_t)((r >> 8) & 1 ? 0x8000 : 0x0000);
    case 1: return (uint16_t)(((r >> 8) & 0x8000) | ((r >> 20) % 127 + 1));     /* subnormal */
    case 2: return (uint16_t)(((r >> 8) & 0x8000) | 0x7F7F);                    /* largest finite */
    default: {
        uint16_t e = (uint16_t)((r >> 12) % 254 + 1), m = (uint16_t)((r >> 24) & 0x7F);
        return (uint16_t)(((r >> 8) & 0x8000) | (e << 7) | m);
    }
    }
}

static void *xcalloc(size_t n, size_t sz) { void *p = calloc(n ? n : 1, sz); if (!p) abort(); return p; }

static int32_t *protected_set(int64_t K, int32_t k)
{
    int32_t *idx = xcalloc((size_t)k, sizeof(int32_t));
    /* k distinct ascending channels spread over [0, K) */
    for (int32_t i = 0; i < k; i++) idx[i] = (int32_t)((int64_t)i * K / (k ? k : 1));
    return idx;
}

static void codecs(void)
{
    for (int n = 0; n < 16; n++) CHECK(oracle_e2m1_round(fabs(oracle_e2m1_decode((uint8_t)n))) == (n & 7));
    for (int b = 0; b < 127; b++) CHECK(oracle_e4m3_round(oracle_e4m3_decode((uint8_t)b)) == b);
    CHECK(oracle_e4m3_round(1e30) == 0x7E);
    CHECK(oracle_e2m1_round(1e30) == 7);
    CHECK(oracle_alpha_from_amax(0.0f) == 1.0f);
    for (uint32_t b = 0; b < 0x10000; b++) {
        const double v = oracle_bf16_to_double((uint16_t)b);
        if (isfinite(v)) CHECK(v == v);
    }
}

/* quantize, dequantize and both GEMMs on one shape */
static void gemm_shape(int64_t M, int64_t N, int64_t K, int32_t k, int64_t pad)
{
    const int64_t ldx = K + pad, ldw = K + pad;
    uint16_t *X = xcalloc((size_t)(M * ldx), 2), *W = xcalloc((size_t)(N * ldw), 2);
    for (int64_t i = 0; i < M * ldx; i++) X[i] = any_bf16();
    for (int64_t i = 0; i < N * ldw; i++) W[i] = any_bf16();
    if (M > 1) memset(X + ldx, 0, (size_t)K * 2);      /* an all-zero row */
    int32_t *idx = protected_set(K, k);
    float ax = 0, aw = 0;
    CHECK(oracle_compute_alpha(X, M, K, ldx, idx, k, &ax) == 0);
    CHECK(oracle_compute_alpha(W, N, K, ldw, idx, k, &aw) == 0);
    CHECK(ax > 0 && aw > 0 && isfinite(ax) && isfinite(aw));
    uint8_t *xq = xcalloc((size_t)(M * K / 2), 1), *xs = xcalloc((size_t)(M * K / 16), 1);
    uint8_t *wq = xcalloc((size_t)(N * K / 2), 1), *ws = xcalloc((size_t)(N * K / 16), 1);
    uint16_t *xS = xcalloc((size_t)(M * k), 2), *wS = xcalloc((size_t)(N * k), 2);
    CHECK(oracle_quantize_nvfp4(X, M, K, ldx, idx, k, ax, xq, xs, k ? xS : NULL) == 0);
    CHECK(oracle_quantize_nvfp4(W, N, K, ldw, idx, k, aw, wq, ws, k ? wS : NULL) == 0);
    for (int64_t i = 0; i < M * K / 16; i++) CHECK(xs[i] <= 0x7E);
    double *dq = xcalloc((size_t)(M * K), sizeof(double));
    CHECK(oracle_dequantize(xq, xs, ax, M, K, dq) == 0);
    for (int64_t i = 0; i < M * K; i++) CHECK(isfinite(dq[i]));
    const int64_t ldy = N + 3;
    float *Y = xcalloc((size_t)(M * ldy), sizeof(float)), *Yn = xcalloc((size_t)(M * ldy), sizeof(float));
    CHECK(oracle_splice_gemm(xq, xs, ax, k ? xS : NULL, wq, ws, aw, k ? wS : NULL, M, N, K, k, Y, ldy) == 0);
    CHECK(oracle_nvfp4_gemm(xq, xs, ax, wq, ws, aw, M, N, K, Yn, ldy) == 0);
    if (k == 0)
        for (int64_t i = 0; i < M * ldy; i++) CHECK(memcmp(&Y[i], &Yn[i], sizeof(float)) == 0);
    float *Yb = xcalloc((size_t)(M * N), sizeof(float));
    double *Yb64 = xcalloc((size_t)(M * N), sizeof(double));
    CHECK(oracle_bf16_gemm(X, W, M, N, K, ldx, ldw, Yb, Yb64) == 0);
    free(X); free(W); free(idx); free(xq); free(xs); free(wq); free(ws); free(xS); free(wS);
    free(dq); free(Y); free(Yn); free(Yb); free(Yb64);
}

static void selection(int64_t T, int64_t K, int32_t k, int64_t stride_rows)
{
    const int64_t ldx = K * stride_rows;
    uint16_t *X = xcalloc((size_t)(T * ldx), 2);
    for (int64_t i = 0; i < T * ldx; i++) X[i] = any_bf16();
    int64_t count = 0;
    double *mean = xcalloc((size_t)K, sizeof(double)), *m2 = xcalloc((size_t)K, sizeof(double));
    float *absmax = xcalloc((size_t)K, sizeof(float));
    int32_t *idx = xcalloc((size_t)k, sizeof(int32_t));
    float alpha = 0;
    CHECK(oracle_select_channels(X, T, K, ldx, k, &count, mean, m2, absmax, idx, &alpha) == 0);
    CHECK(count == T);
    for (int32_t i = 1; i < k; i++) CHECK(idx[i] > idx[i - 1]);
    /* a second fold of the same rows, then the second-moment ranking */
    CHECK(oracle_stats(X, T, K, ldx, &count, mean, m2, absmax) == 0);
    double *sm = xcalloc((size_t)K, sizeof(double));
    CHECK(oracle_second_moments(mean, m2, count, K, sm) == 0);
    CHECK(oracle_select_topk(sm, K, k, idx) == 0);
    CHECK(oracle_alpha_from_absmax(absmax, K, idx, k, &alpha) == 0);
    free(X); free(mean); free(m2); free(absmax); free(idx); free(sm);
}

static void tim(int64_t B, int64_t L)
{
    float *logp = xcalloc((size_t)(B * L), sizeof(float)), *adv = xcalloc((size_t)(B * 3), sizeof(float));
    int32_t *len = xcalloc((size_t)B, sizeof(int32_t)), *g1 = xcalloc((size_t)B, 4), *g2 = xcalloc((size_t)B, 4);
    uint8_t *keep = xcalloc((size_t)B, 1);
    for (int64_t i = 0; i < B * L; i++) logp[i] = -(float)(next_u64() % 2000) / 100.0f;
    for (int64_t b = 0; b < B; b++) len[b] = (int32_t)(b == 0 ? 0 : (b == 1 ? L : (int64_t)(next_u64() % (L + 1))));
    for (int64_t i = 0; i < B * 3; i++) adv[i] = 1.0f;
    CHECK(oracle_tim_filter(logp, B, L, len, -9.21f, 1, 100, 5, keep, g1, g2, adv, 3, 3) == 0);
    for (int64_t b = 0; b < B; b++) CHECK(keep[b] <= 1 && g1[b] >= 0 && g2[b] >= 0 && g2[b] <= g1[b]);
    free(logp); free(adv); free(len); free(g1); free(g2); free(keep);
}

int main(void)
{
    codecs();
    /* (M, N, K, k, row padding): one block, k = 0, k = K, ragged, padded rows */
    const int64_t shapes[][5] = {{1, 1, 16, 0, 0}, {1, 1, 16, 16, 0}, {3, 5, 48, 7, 5}, {4, 2, 64, 64, 0},
                                 {7, 9, 128, 3, 16}, {2, 3, 256, 0, 1}, {0, 4, 32, 2, 0}, {5, 0, 32, 2, 0}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); i++)
        gemm_shape(shapes[i][0], shapes[i][1], shapes[i][2], (int32_t)shapes[i][3], shapes[i][4]);
    selection(1, 16, 1, 1);
    selection(70, 48, 5, 2);
    selection(130, 256, 64, 1);
    tim(6, 40);
    /* argument errors are reported, not acted on */
    float a = 0;
    int32_t bad[2] = {3, 3};
    uint16_t z[32] = {0};
    CHECK(oracle_compute_alpha(z, 1, 32, 32, bad, 2, &a) != 0);
    CHECK(oracle_dequantize(NULL, NULL, 1.0f, 1, 17, NULL) != 0);
    CHECK(oracle_select_topk(NULL, 4, 5, NULL) != 0);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
