/*
 * oracle.c -- plain, slow, fp64 CPU oracle for SpliceGEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__
 * and the cpu_baseline leg of bench.py may load this library.  It shares no
 * code, header, table or helper with the HIP path in fp4_gemm_sparse_amd/.
 *
 * What it computes follows the FourSight paper ("FourSight: Stable FP4 RL
 * Post-Training via Sequence Filtering and Sparse Channel Compensation",
 * arXiv 2611.04887v1):
 *   - NVFP4: E2M1 elements in 16-element blocks along the reduction dim, one
 *     E4M3 scale per block, one FP32 tensor scale                (Sec. 2.1)
 *   - protected channels S are zeroed before the block scales are computed,
 *     so the block scales are recomputed on the residual          (App. 9.3.1)
 *   - block scale s_b = round_E4M3(g * a_b / 6) / g               (App. 9.3.1, Eq. 9)
 *   - Y = alpha_X alpha_W * deq(Q(X_R)) deq(Q(W_R))^T + X_S W_S^T (Sec. 4.2 Eq. 5,
 *                                                                  App. 9.3.1 Eq. 7-8)
 *   - top-s variance channel selection                            (Sec. 4.2)
 *   - top-s second-moment selection, the minimiser of the relaxed
 *     error bound                                    (App., Prop. 2, Cor. 1)
 *   - TIM-aware sequence filtering: tail tokens, the cumulative gate G1,
 *     the consecutive gate G2 and the masked advantages (Sec. 4.1, Eq. 3-4)
 *   - running channel moments accumulated from token rows         (Sec. 5.2)
 *
 * Conventions the pages leave open and that this oracle fixes (each one is
 * a reading of an open point, not something the pages state):
 *   - g = 1/alpha with alpha = fp32(masked amax / (6*448)); alpha = 1 when the
 *     masked tensor is all zero.
 *   - the E4M3 variant is OCP E4M3FN (max 448, no infinities); rounding of the
 *     scale is round-to-nearest-even on the exact real a_b/(6 alpha), with
 *     saturation at 448; subnormal scales are allowed.
 *   - element rounding is round-to-nearest on the exact real |x|/(s_b alpha)
 *     onto {0,0.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6;
 *     the nibble keeps the sign bit of x (so -0 and tiny negatives give 0x8);
 *     protected lanes are +0 and give 0x0.
 *   - codes are packed two per byte, the even channel in the low nibble;
 *     scales are row-major [R, K/16] bytes; side buffers hold the protected
 *     columns in ascending channel order, copied bit for bit.
 *   - statistics: Welford (1962) inside 64-row tiles, then the pairwise
 *     update of Chan, Golub & LeVeque (1983) folding tiles left to right.
 *   - selection ranks by M2 (n is the same for every channel), larger first,
 *     ties to the lower channel index; the result is returned ascending.
 *   - the second moment of a channel is formed from the running moments as
 *     m2/n + mean*mean (variance plus squared mean, three roundings), 0 when
 *     no row has been seen; it is ranked the same way.
 *
 * Every fp64 expression is written so that each operator is one IEEE
 * rounding; the file is compiled with -ffp-contract=off.
 *
 * Why the fp64 quotients decide the roundings exactly: a_b and |x| are bf16
 * (8 significant bits), alpha is fp32 (24), an E4M3 value has 4 and a
 * rounding midpoint at most 5 significant bits, so an exact real quotient
 * either equals a midpoint (then the fp64 quotient is that midpoint exactly)
 * or differs from it by more than 2^-40 relative, far above the 2^-53
 * relative error of one fp64 division.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLOCK 16
#define STATS_TILE_ROWS 64

/* ------------------------------------------------------------------ */
/* bf16 bit patterns                                                  */
/* ------------------------------------------------------------------ */

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* E2M1 (Sec. 2.1; value set stated in App. 9.3.1)                    */
/* ------------------------------------------------------------------ */

/* magnitude of code c = 0..7 */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* signed value of a 4-bit code: bit 3 is the sign */
double oracle_e2m1_decode(uint8_t nibble)
{
    double m = E2M1_MAG[nibble & 7];
    return (nibble & 8) ? -m : m;
}

/* Round r >= 0 to the nearest E2M1 magnitude, ties to the even code,
 * saturating at 6.  Returns the 3-bit magnitude code. */
uint8_t oracle_e2m1_round(double r)
{
    if (r >= 6.0) return 7;
    int lo = 0;
    while (lo < 7 && E2M1_MAG[lo + 1] <= r) lo++;   /* E2M1_MAG[lo] <= r < E2M1_MAG[lo+1] */
    double mid = (E2M1_MAG[lo] + E2M1_MAG[lo + 1]) * 0.5;  /* exact */
    if (r < mid) return (uint8_t)lo;
    if (r > mid) return (uint8_t)(lo + 1);
    return (lo % 2 == 0) ? (uint8_t)lo : (uint8_t)(lo + 1);
}

/* ------------------------------------------------------------------ */
/* E4M3FN (OCP FP8): 1 sign, 4 exponent (bias 7), 3 mantissa bits;     */
/* exponent field 15 with mantissa 7 is NaN; max finite 448.          */
/* ------------------------------------------------------------------ */

double oracle_e4m3_decode(uint8_t b)
{
    int e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                 /* subnormal m * 2^-9 */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (b & 0x80) ? -v : v;
}

/* Round v >= 0 to the nearest non-negative finite E4M3FN value, ties to the
 * even mantissa, saturating at 448.  Non-negative finite codes 0x00..0x7E
 * are increasing in value, so the neighbours are found by a scan. */
uint8_t oracle_e4m3_round(double v)
{
    if (v >= 448.0) return 0x7E;
    int lo = 0;
    while (lo < 0x7E && oracle_e4m3_decode((uint8_t)(lo + 1)) <= v) lo++;
    double a = oracle_e4m3_decode((uint8_t)lo), b = oracle_e4m3_decode((uint8_t)(lo + 1));
    double mid = (a + b) * 0.5;                           /* exact: few bits */
    if (v < mid) return (uint8_t)lo;
    if (v > mid) return (uint8_t)(lo + 1);
    return (lo % 2 == 0) ? (uint8_t)lo : (uint8_t)(lo + 1);
}

/* ------------------------------------------------------------------ */
/* helpers over the protected set                                     */
/* ------------------------------------------------------------------ */

/* 1 for protected channels, 0 otherwise; idx must be strictly ascending. */
static unsigned char *protected_flags(int64_t K, const int32_t *idx, int32_t k)
{
    unsigned char *p = (unsigned char *)calloc((size_t)(K > 0 ? K : 1), 1);
    for (int32_t i = 0; i < k; i++) p[idx[i]] = 1;
    return p;
}

static int idx_valid(int64_t K, const int32_t *idx, int32_t k)
{
    if (k < 0 || k > K) return 0;
    for (int32_t i = 0; i < k; i++) {
        if (idx[i] < 0 || idx[i] >= K) return 0;
        if (i > 0 && idx[i] <= idx[i - 1]) return 0;
    }
    return 1;
}

/* ------------------------------------------------------------------ */
/* Global scale alpha: one FP32 scale per tensor (Sec. 2.1); it is    */
/* the inverse of the encode gain g of App. 9.3.1 Eq. 9.              */
/* ------------------------------------------------------------------ */

float oracle_alpha_from_amax(float amax)
{
    if (amax == 0.0f) return 1.0f;
    return amax / 2688.0f;             /* one correctly rounded fp32 division */
}

/* alpha of the masked matrix A[R,K] (row stride lda): protected columns are
 * left out of the maximum.  Returns -1 on bad arguments. */
int oracle_compute_alpha(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                         const int32_t *idx, int32_t k, float *alpha)
{
    if (R < 0 || K < 0 || lda < K || !idx_valid(K, idx, k)) return -1;
    unsigned char *prot = protected_flags(K, idx, k);
    double amax = 0.0;
    for (int64_t r = 0; r < R; r++)
        for (int64_t j = 0; j < K; j++) {
            if (prot[j]) continue;
            double a = fabs(oracle_bf16_to_double(A[r * lda + j]));
            if (a > amax) amax = a;
        }
    free(prot);
    *alpha = oracle_alpha_from_amax((float)amax);   /* amax is a bf16 value: exact */
    return 0;
}

/* alpha from per-channel absmax statistics (the frozen activation scale of
 * a warm-up batch): max over unprotected channels. */
int oracle_alpha_from_absmax(const float *absmax, int64_t K, const int32_t *idx, int32_t k,
                             float *alpha)
{
    if (K < 0 || !idx_valid(K, idx, k)) return -1;
    unsigned char *prot = protected_flags(K, idx, k);
    float amax = 0.0f;
    for (int64_t j = 0; j < K; j++)
        if (!prot[j] && absmax[j] > amax) amax = absmax[j];
    free(prot);
    *alpha = oracle_alpha_from_amax(amax);
    return 0;
}

/* ------------------------------------------------------------------ */
/* NVFP4 quantization of the masked residual (Sec. 5.1 data           */
/* preparation; App. 9.3.1 Eq. 9) plus the gather of the protected    */
/* columns into a compact side buffer.                                 */
/* ------------------------------------------------------------------ */

int oracle_quantize_nvfp4(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                          const int32_t *idx, int32_t k, float alpha,
                          uint8_t *codes, uint8_t *scales, uint16_t *side)
{
    if (R < 0 || K < 0 || K % BLOCK != 0 || lda < K || !idx_valid(K, idx, k)) return -1;
    if (!(alpha > 0.0f) || isinf(alpha)) return -1;
    unsigned char *prot = protected_flags(K, idx, k);
    const int64_t nb = K / BLOCK;
    const double six_alpha = 6.0 * (double)alpha;       /* exact */

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        for (int64_t b = 0; b < nb; b++) {
            double x[BLOCK];
            double a_b = 0.0;
            for (int t = 0; t < BLOCK; t++) {
                int64_t j = b * BLOCK + t;
                x[t] = prot[j] ? 0.0 : oracle_bf16_to_double(A[r * lda + j]);  /* mask S -> +0 */
                if (fabs(x[t]) > a_b) a_b = fabs(x[t]);
            }
            uint8_t sc = oracle_e4m3_round(a_b / six_alpha);
            double s = oracle_e4m3_decode(sc);
            double phys = s * (double)alpha;                   /* exact: 4 x 24 bits */
            scales[r * nb + b] = sc;
            for (int t = 0; t < BLOCK; t += 2) {
                uint8_t nib[2];
                for (int u = 0; u < 2; u++) {
                    double v = x[t + u];
                    uint8_t c = (s == 0.0) ? 0 : oracle_e2m1_round(fabs(v) / phys);
                    nib[u] = (uint8_t)((signbit(v) ? 8 : 0) | c);
                }
                codes[r * (K / 2) + (b * BLOCK + t) / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
            }
        }
        for (int32_t i = 0; i < k; i++) side[r * (int64_t)k + i] = A[r * lda + idx[i]];
    }
    free(prot);
    return 0;
}

/* The real value each quantized element stands for: alpha * e2m1 * scale. */
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float alpha,
                      int64_t R, int64_t K, double *out)
{
    if (R < 0 || K < 0 || K % BLOCK != 0) return -1;
    for (int64_t r = 0; r < R; r++)
        for (int64_t j = 0; j < K; j++) {
            uint8_t byte = codes[r * (K / 2) + j / 2];
            uint8_t nib = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
            double s = oracle_e4m3_decode(scales[r * (K / BLOCK) + j / BLOCK]);
            out[r * K + j] = oracle_e2m1_decode(nib) * s * (double)alpha;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* GEMMs (Sec. 4.2 Eq. 5; App. 9.3.1 Eq. 8)                            */
/* ------------------------------------------------------------------ */

/* Y[m,n] = fp32( alpha_x*alpha_w * sum_k deq(X)[m,k] deq(W)[n,k]  +  sum_i X_S[m,i] W_S[n,i] )
 * Both sums in fp64, in increasing k and i.  Every product of two decoded
 * NVFP4 values is exact in fp64 (6 x 6 significant bits), as is every bf16
 * product.  k == 0 gives the plain NVFP4 product. */
int oracle_splice_gemm(const uint8_t *Xq, const uint8_t *Xs, float alpha_x, const uint16_t *X_S,
                       const uint8_t *Wq, const uint8_t *Ws, float alpha_w, const uint16_t *W_S,
                       int64_t M, int64_t N, int64_t K, int32_t k, float *Y, int64_t ldy)
{
    if (M < 0 || N < 0 || K < 0 || K % BLOCK != 0 || k < 0 || k > K || ldy < N) return -1;
    const int64_t nb = K / BLOCK;
    const double alpha = (double)alpha_x * (double)alpha_w;   /* exact: 24 x 24 bits */

    /* decoded operands without alpha (exact): e2m1 * e4m3 */
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *wd = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    for (int64_t m = 0; m < M; m++)
        for (int64_t j = 0; j < K; j++) {
            uint8_t byte = Xq[m * (K / 2) + j / 2];
            uint8_t nib = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
            xd[m * K + j] = oracle_e2m1_decode(nib) * oracle_e4m3_decode(Xs[m * nb + j / BLOCK]);
        }
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < K; j++) {
            uint8_t byte = Wq[n * (K / 2) + j / 2];
            uint8_t nib = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
            wd[n * K + j] = oracle_e2m1_decode(nib) * oracle_e4m3_decode(Ws[n * nb + j / BLOCK]);
        }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            double acc4 = 0.0;
            for (int64_t j = 0; j < K; j++) acc4 += xd[m * K + j] * wd[n * K + j];
            double accS = 0.0;
            for (int32_t i = 0; i < k; i++)
                accS += oracle_bf16_to_double(X_S[m * (int64_t)k + i]) *
                        oracle_bf16_to_double(W_S[n * (int64_t)k + i]);
            Y[m * ldy + n] = (float)(acc4 * alpha + accS);
        }
    }
    free(xd);
    free(wd);
    return 0;
}

int oracle_nvfp4_gemm(const uint8_t *Xq, const uint8_t *Xs, float alpha_x,
                      const uint8_t *Wq, const uint8_t *Ws, float alpha_w,
                      int64_t M, int64_t N, int64_t K, float *Y, int64_t ldy)
{
    return oracle_splice_gemm(Xq, Xs, alpha_x, NULL, Wq, Ws, alpha_w, NULL, M, N, K, 0, Y, ldy);
}

/* The unquantized product Y = X W^T of bf16 operands, summed in fp64 in
 * increasing k; Y64 (may be NULL) receives the fp64 sums, Y (may be NULL)
 * their fp32 rounding. */
int oracle_bf16_gemm(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N, int64_t K,
                     int64_t ldx, int64_t ldw, float *Y, double *Y64)
{
    if (M < 0 || N < 0 || K < 0 || ldx < K || ldw < K) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t j = 0; j < K; j++)
                acc += oracle_bf16_to_double(X[m * ldx + j]) * oracle_bf16_to_double(W[n * ldw + j]);
            if (Y) Y[m * N + n] = (float)acc;
            if (Y64) Y64[m * N + n] = acc;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Channel statistics (Sec. 5.2: running channel moments from token   */
/* rows) and top-s selection by activation variance (Sec. 4.2).      */
/* ------------------------------------------------------------------ */

typedef struct { double n, mean, m2; } moments;

/* Chan, Golub & LeVeque pairwise update, left operand first. */
static moments chan_merge(moments a, moments b)
{
    if (b.n == 0.0) return a;
    if (a.n == 0.0) return b;
    moments r;
    double n = a.n + b.n;
    double d = b.mean - a.mean;
    r.n = n;
    r.mean = a.mean + d * (b.n / n);
    r.m2 = a.m2 + b.m2 + (d * d) * (a.n * b.n / n);
    return r;
}

/* Accumulate the T rows of X[T,K] (row stride ldx) into running per-channel
 * moments.  *count (host) is the number of rows already folded in; 0 means
 * the running buffers are ignored and overwritten.  The batch is split into
 * 64-row tiles; each tile is a Welford pass in row order; tiles are folded
 * left to right; the batch is then folded into the running moments. */
int oracle_stats(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int64_t *count,
                 double *mean, double *m2, float *absmax)
{
    if (T < 0 || K < 0 || ldx < K || *count < 0) return -1;
    const int64_t n_prev = *count;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; j++) {
        moments acc = {0.0, 0.0, 0.0};
        double amax = 0.0;
        for (int64_t t0 = 0; t0 < T; t0 += STATS_TILE_ROWS) {
            int64_t t1 = t0 + STATS_TILE_ROWS < T ? t0 + STATS_TILE_ROWS : T;
            moments tile = {0.0, 0.0, 0.0};
            for (int64_t t = t0; t < t1; t++) {
                double x = oracle_bf16_to_double(X[t * ldx + j]);
                tile.n += 1.0;
                double d = x - tile.mean;
                tile.mean += d / tile.n;
                tile.m2 += d * (x - tile.mean);
                if (fabs(x) > amax) amax = fabs(x);
            }
            acc = chan_merge(acc, tile);
        }
        moments run = {0.0, 0.0, 0.0};
        float prev_amax = 0.0f;
        if (n_prev > 0) {
            run.n = (double)n_prev;
            run.mean = mean[j];
            run.m2 = m2[j];
            prev_amax = absmax[j];
        }
        run = chan_merge(run, acc);
        mean[j] = run.mean;
        m2[j] = run.m2;
        absmax[j] = (float)amax > prev_amax ? (float)amax : prev_amax;
    }
    *count = n_prev + T;
    return 0;
}

static const double *g_sort_key;
static int key_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    if (g_sort_key[a] > g_sort_key[b]) return -1;   /* larger M2 first */
    if (g_sort_key[a] < g_sort_key[b]) return 1;
    return (a < b) ? -1 : (a > b);                  /* tie: lower index first */
}
static int int_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a < b) ? -1 : (a > b);
}

/* idx[0..k) = the k channels with the largest m2 (ties to the lower index),
 * returned in ascending channel order. */
int oracle_select_topk(const double *m2, int64_t K, int32_t k, int32_t *idx)
{
    if (K < 0 || k < 0 || k > K) return -1;
    for (int64_t j = 0; j < K; j++)
        if (isnan(m2[j])) return -1;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    for (int64_t j = 0; j < K; j++) order[j] = (int32_t)j;
    g_sort_key = m2;
    qsort(order, (size_t)K, sizeof(int32_t), key_cmp);
    memcpy(idx, order, sizeof(int32_t) * (size_t)k);
    qsort(idx, (size_t)k, sizeof(int32_t), int_cmp);
    free(order);
    return 0;
}

/* Second moments m_j = E[x_j^2] of K channels from running moments over n
 * rows: the population variance m2_j / n plus the squared mean (the relaxed
 * bound of Prop. 2 is minimised by the largest m_j; Cor. 1 says when the
 * largest variances give the same set).  0 for every channel when n == 0. */
int oracle_second_moments(const double *mean, const double *m2, int64_t n, int64_t K, double *out)
{
    if (n < 0 || K < 0) return -1;
    for (int64_t j = 0; j < K; j++) {
        if (n == 0) {
            out[j] = 0.0;
            continue;
        }
        double v = m2[j] / (double)n;
        double mu2 = mean[j] * mean[j];
        out[j] = v + mu2;
    }
    return 0;
}

/* Statistics, selection and the frozen activation scale in one call, the
 * calibration step that chooses S for a projection. */
int oracle_select_channels(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int32_t k,
                           int64_t *count, double *mean, double *m2, float *absmax,
                           int32_t *idx, float *alpha_x)
{
    int rc = oracle_stats(X, T, K, ldx, count, mean, m2, absmax);
    if (rc) return rc;
    rc = oracle_select_topk(m2, K, k, idx);
    if (rc) return rc;
    if (alpha_x) rc = oracle_alpha_from_absmax(absmax, K, idx, k, alpha_x);
    return rc;
}

/* ------------------------------------------------------------------ */
/* TIM-aware sequence filtering (Sec. 4.1, Eq. 3-4; settings Sec. 6.1) */
/* ------------------------------------------------------------------ */

/* For each of B sequences: token t < len[i] is a tail token when its
 * training-policy log-probability logp[i*ldl + t] <= log_tau (pi_train <= tau
 * in the log domain; tokens at or past len[i] are padding).
 *   G1 = number of tail tokens, G2 = longest run of consecutive tail tokens;
 *   the sequence is kept (f_i = 1) when G1 < K1 and G2 < K2 with
 *   K1 = (k1_num / k1_den) * len[i], compared exactly as
 *   G1 * k1_den < k1_num * len[i];
 *   adv[i*lda + c] for c < adv_cols is multiplied by f_i: a dropped
 *   sequence's advantages become +0, a kept one's are untouched (Eq. 4).
 * keep, g1, g2 and adv may each be NULL. */
int oracle_tim_filter(const float *logp, int64_t B, int64_t ldl, const int32_t *len,
                      float log_tau, int64_t k1_num, int64_t k1_den, int64_t k2,
                      uint8_t *keep, int32_t *g1, int32_t *g2,
                      float *adv, int64_t adv_cols, int64_t lda)
{
    if (B < 0 || k1_num < 0 || k1_den <= 0 || k2 < 0 || adv_cols < 0) return -1;
    for (int64_t i = 0; i < B; i++) {
        const int64_t n = len[i];
        if (n < 0 || n > ldl) return -1;
        int64_t count = 0, run = 0, longest = 0;
        for (int64_t t = 0; t < n; t++) {
            if (logp[i * ldl + t] <= log_tau) {
                count++;
                run++;
                if (run > longest) longest = run;
            } else {
                run = 0;
            }
        }
        const int kept = (count * k1_den < k1_num * n) && (longest < k2);
        if (keep) keep[i] = (uint8_t)kept;
        if (g1) g1[i] = (int32_t)count;
        if (g2) g2[i] = (int32_t)longest;
        if (adv && !kept)
            for (int64_t c = 0; c < adv_cols; c++) adv[i * lda + c] = 0.0f;
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
