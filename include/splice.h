/*
 * splice.h -- C ABI of libsplice.so, SpliceGEMM on AMD Instinct MI355X (gfx950).
 *
 * SpliceGEMM is the W4A4 NVFP4 linear layer of the FourSight paper
 * (arXiv 2611.04887v1, Sec. 4.2 and 5.1): the K input channels are split into
 * a small protected set S, kept in BF16, and its complement, quantized to NVFP4
 * after the protected coordinates are set to zero (App. 9.3.1):
 *
 *     Y = alpha_X * alpha_W * deq(Xq) deq(Wq)^T  +  X_S W_S^T        (fp32)
 *
 * Number formats (NVFP4, Sec. 2.1):
 *   codes   uint8 [R, K/2]   E2M1 nibbles, channel 2i in the low nibble of
 *                            byte i; nibble = sign<<3 | magnitude code, the
 *                            magnitude codes 0..7 standing for 0, 0.5, 1, 1.5,
 *                            2, 3, 4, 6
 *   scales  uint8 [R, K/16]  one OCP E4M3FN byte per 16-channel block
 *                            (non-negative, finite), row-major
 *   alpha   float            FP32 tensor scale (a decode scale: value =
 *                            alpha * e2m1 * e4m3), passed as a DEVICE pointer
 *   side    bf16  [R, k]     the protected columns A[:, idx[i]], bit for bit
 *   bf16 tensors are passed as uint16_t bit patterns.
 *
 * Quantization rule (App. 9.3.1 Eq. 9 with encode gain 1/alpha; round-to-
 * nearest-even decisions taken on exact real quotients):
 *   a_b = max |x_j| over the block, protected lanes counted as +0
 *   s_b = E4M3FN(a_b / (6 alpha)), ties to even, saturating at 448
 *   code = nearest E2M1 magnitude to |x| / (s_b alpha), ties to the even code,
 *          saturating at 6; 0 when s_b = 0; protected lanes give nibble 0
 *   alpha (splice_compute_alpha, splice_select_channels) = fp32(amax / 2688)
 *          over the unprotected entries, 1 when that maximum is 0
 *
 * General rules for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller unless marked HOST.  The
 *     library allocates and frees nothing; scratch comes in through `ws`.
 *   - Work is enqueued on `stream` (0 = the null stream) and is asynchronous.
 *     Argument errors are detected on the host and returned synchronously
 *     before anything is enqueued; a launch failure returns SPLICE_ERR_HIP.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Shapes: K % 16 == 0 (NVFP4 block), 0 <= k <= K, K <= 65536,
 *     M, N, R, T >= 0 (zero sizes are no-ops).  idx holds k strictly
 *     ascending channel indices in [0, K) (a DEVICE array; its order is the
 *     caller's contract and is not checked).
 *   - Row strides (lda, ldx, ldy) are in elements and must be >= the row
 *     length.  Buffers must be 16-byte aligned.
 *   - Functions are stateless and thread-safe; calls that share output or
 *     workspace buffers must be ordered by the caller.
 *   - Results do not depend on the path taken or the launch configuration
 *     except for fp32 rounding order in the GEMM accumulators.
 *   - Logging: with SPLICE_LOG set to anything but "" or "0" in the
 *     environment when the library is first used, every GEMM call
 *     (splice_gemm, splice_gemm_noalloc, nvfp4_gemm, splice_gemm_multi) that
 *     passes its argument checks writes one line to stderr: its shape, the
 *     path, kernel, tile and K split its plan chose (as splice_gemm_plan
 *     reports them) and the status it returns.
 *   - Profiler ranges: with SPLICE_ROCTX set to anything but "" or "0" when
 *     the library is first used, every compute entry point runs inside a
 *     roctx range named for the function and its shape (for example
 *     "splice_gemm M=128 N=4096 K=4096 k=64"), which marker traces such as
 *     rocprofv3 --marker-trace line up with the kernels the call launched.
 *     The roctx library is opened at that first use, so linking against this
 *     library needs no roctx; when it cannot be opened, calls run unmarked.
 */
#ifndef SPLICE_H
#define SPLICE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *splice_stream_t;   /* == hipStream_t */

typedef enum {
    SPLICE_OK = 0,
    SPLICE_ERR_INVALID_ARG = -1,   /* bad pointer, size, stride or alignment */
    SPLICE_ERR_UNSUPPORTED = -2,   /* valid but outside what the kernels handle */
    SPLICE_ERR_WORKSPACE = -3,     /* ws too small (see the *_workspace_size calls) */
    SPLICE_ERR_HIP = -4            /* the HIP runtime reported an error */
} splice_status;

enum { SPLICE_PATH_AUTO = 0, SPLICE_PATH_DECODE = 1, SPLICE_PATH_PREFILL = 2 };

/* Largest M the automatic dispatch sends to the decode (weight-streaming)
 * path.  The paper switches at 32 tokens (Sec. 5.1); the decode kernels here
 * take up to 64 rows. */
#define SPLICE_DECODE_MAX_M 64

/* Human-readable name of a status code (static string). */
const char *splice_status_string(int status);

/* ---------------------------------------------------------------------------
 * Channel statistics and top-k selection (Sec. 4.2 variance-based selection;
 * Sec. 5.2 running channel moments from token rows).
 *
 * Folds the T rows of X (bf16 [T, K], row stride ldx -- a stride that is a
 * multiple of K subsamples rows) into running per-channel moments, then
 * selects the k channels with the largest M2 (equivalently the largest
 * variance: every channel has the same count), ties to the lower index,
 * written to idx[0..k) in ascending order.
 *   count   HOST in/out: rows already folded into mean/m2/absmax; 0 means the
 *           running buffers are ignored and overwritten.  Updated to count+T.
 *   mean, m2  double [K] in/out (sum of squared deviations)
 *   absmax  float [K] in/out
 *   idx     int32 [k] out
 *   alpha_x float [1] out (may be NULL): the frozen activation scale
 *           fp32(max over unprotected channels of absmax / 2688), 1 if 0.
 * Arithmetic: Welford inside 64-row tiles, tiles folded left to right with the
 * pairwise update of Chan, Golub & LeVeque, then merge(running, batch); every
 * step in fp64 with one IEEE rounding per operation, so the result is
 * bit-identical to a sequential evaluation in that order.
 * ws: splice_select_workspace_size(K) bytes. */
int splice_select_channels(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int32_t k,
                           int64_t *count, double *mean, double *m2, float *absmax,
                           int32_t *idx, float *alpha_x,
                           void *ws, size_t ws_bytes, splice_stream_t stream);
size_t splice_select_workspace_size(int64_t K);

/* ---------------------------------------------------------------------------
 * The two halves of splice_select_channels, for callers that fold token rows
 * into the running moments as they pass (Sec. 5.2: a forward hook subsamples
 * rows into running channel moments; the protected set is reselected once
 * per optimizer step from what the previous step gathered).
 *
 * splice_channel_stats: folds the T rows of X into mean/m2/absmax exactly as
 * splice_select_channels does (same arguments, same arithmetic, same count
 * rules), without selecting.
 *
 * splice_select_topk: the k channels ranked by `criterion` from running
 * moments over `count` rows (count is a HOST value), ties to the lower index,
 * written to idx[0..k) ascending, and alpha_x (may be NULL) as for
 * splice_select_channels.
 *   SPLICE_SELECT_VARIANCE: the largest M2 (the paper's selection, Sec. 4.2);
 *     mean may be NULL.
 *   SPLICE_SELECT_SECOND_MOMENT: the largest m2/count + mean^2 = E[x^2] per
 *     channel (fp64, one rounding per operation; 0 when count == 0), the set
 *     that minimises the relaxed error bound (App. Prop. 2); Cor. 1 gives the
 *     condition on the means under which both criteria pick the same set. */
enum { SPLICE_SELECT_VARIANCE = 0, SPLICE_SELECT_SECOND_MOMENT = 1 };
int splice_channel_stats(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int64_t *count,
                         double *mean, double *m2, float *absmax, splice_stream_t stream);
int splice_select_topk(const double *mean, const double *m2, const float *absmax, int64_t count,
                       int64_t K, int32_t k, int criterion, int32_t *idx, float *alpha_x,
                       splice_stream_t stream);

/* ---------------------------------------------------------------------------
 * alpha = fp32(max |A| over the unprotected columns / 2688), 1 if that is 0
 * (Sec. 2.1 FP32 tensor scale; App. 9.3.1 Eq. 9).  A: bf16 [R, K], stride
 * lda.  alpha: float [1] out.  ws: splice_alpha_workspace_size() bytes. */
int splice_compute_alpha(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                         const int32_t *idx, int32_t k, float *alpha,
                         void *ws, size_t ws_bytes, splice_stream_t stream);
size_t splice_alpha_workspace_size(void);

/* ---------------------------------------------------------------------------
 * Mask, quantize and gather (Sec. 5.1 data preparation; weight pre-split):
 * one pass over A (bf16 [R, K], stride lda) writes the NVFP4 codes and block
 * scales of the masked residual and the protected columns.
 *   alpha  float [1] in (DEVICE), > 0 and finite
 *   codes  uint8 [R, K/2] out;  scales uint8 [R, K/16] out
 *   side   bf16 [R, k] out (may be NULL when k == 0) */
int splice_quantize_nvfp4(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                          const int32_t *idx, int32_t k, const float *alpha,
                          uint8_t *codes, uint8_t *scales, uint16_t *side,
                          splice_stream_t stream);

/* ---------------------------------------------------------------------------
 * SpliceGEMM (Sec. 4.2 Eq. 5; Sec. 5.1 dual-path execution):
 *   Y[m, n] = alpha_x*alpha_w * sum_j deq(Xq)[m, j] deq(Wq)[n, j]
 *             + sum_i X_S[m, i] W_S[n, i]
 * Xq/Xs: [M, K/2] / [M, K/16];  Wq/Ws: [N, K/2] / [N, K/16];
 * X_S: bf16 [M, k], W_S: bf16 [N, k] (unscaled, bit copies of the protected
 * columns); Y: fp32 [M, N] out with row stride ldy.
 * The NVFP4 operands are decoded exactly to FP16 (an E2M1 value times an
 * E4M3 scale has at most 6 significant bits) and multiplied on the FP16
 * matrix cores with fp32 accumulation; the BF16 side product is computed on
 * the BF16 matrix cores and added to alpha_x*alpha_w times that accumulator.
 * path: SPLICE_PATH_AUTO (decode path when M <= SPLICE_DECODE_MAX_M),
 *       SPLICE_PATH_DECODE (requires M <= SPLICE_DECODE_MAX_M) or
 *       SPLICE_PATH_PREFILL.
 * ws: DEVICE workspace of at least splice_workspace_size(M, N, K, k) bytes,
 *     16-byte aligned (NULL is allowed when that size is 0; a smaller or
 *     missing workspace returns SPLICE_ERR_WORKSPACE).  Either path splits
 *     the K range over workgroups when its output tiles alone would leave CUs
 *     idle: the prefill path at small M (up to a few hundred rows), the decode
 *     path for narrow or deep projections (few column groups, or long K).
 *     The workspace then holds one arrival counter per output tile (column
 *     group) and the fp32 partial sums, which the workgroup completing a tile
 *     adds in split order, so Y does not depend on arrival order.  The
 *     counters must be zero when the workspace is first used -- zero-fill it
 *     once after allocating it -- and every call leaves them zero again, so
 *     one workspace serves any sequence of calls ordered on a stream (calls
 *     that may run concurrently need workspaces of their own).  At most
 *     16 MiB + 1 KiB; 0 for large M. */
int splice_gemm(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint16_t *X_S,
                const uint8_t *Wq, const uint8_t *Ws, const float *alpha_w, const uint16_t *W_S,
                int64_t M, int64_t N, int64_t K, int32_t k, float *Y, int64_t ldy,
                void *ws, size_t ws_bytes, int path, splice_stream_t stream);

/* splice_gemm for callers that cannot allocate device memory (code under
 * stream or graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results as splice_gemm (bit for bit), with
 * the workspace taken from a device array the library holds for the life of
 * the process, SPLICE_NOALLOC_SCRATCH_BYTES on every GPU it runs on (the
 * largest workspace any shape needs).  The first call on a device looks the
 * array up and clears its counters on `stream`; no call allocates or frees
 * anything.  Every call on a GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams, different threads) race and must be
 * ordered by the caller.  A shape whose workspace would exceed the array
 * returns SPLICE_ERR_WORKSPACE; other errors as splice_gemm. */
#define SPLICE_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u + 1024u)
int splice_gemm_noalloc(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint16_t *X_S,
                        const uint8_t *Wq, const uint8_t *Ws, const float *alpha_w, const uint16_t *W_S,
                        int64_t M, int64_t N, int64_t K, int32_t k, float *Y, int64_t ldy, int path,
                        splice_stream_t stream);

/* Plain NVFP4 GEMM without compensation, the overhead baseline (the paper's
 * uncompensated FP4, Sec. 6.3): splice_gemm with k = 0. */
int nvfp4_gemm(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x,
               const uint8_t *Wq, const uint8_t *Ws, const float *alpha_w,
               int64_t M, int64_t N, int64_t K, float *Y, int64_t ldy,
               void *ws, size_t ws_bytes, int path, splice_stream_t stream);

/* ---------------------------------------------------------------------------
 * SpliceGEMM for decode with the activation preparation done inside the GEMM
 * (Sec. 5.1 data preparation and dual-path execution; the preparation is
 * part of the projection's cost in Sec. 6.3): the kernel reads the bf16
 * activations, masks the protected channels, quantizes the residual to NVFP4
 * with alpha_x and gathers X_S itself, then computes the splice_gemm product.
 * The same operand bits reach the matrix cores as in the two-call form
 * (splice_quantize_nvfp4(X, idx, alpha_x), then splice_gemm on the decode
 * path): one launch instead of two and no Xq/Xs/X_S buffers.  Y is
 * bit-identical to the two-call form where both use the same chunk split and
 * summation order (K/128 even and M*K <= 32768), and within the GEMM
 * tolerance otherwise.  Every workgroup repeats the preparation of the M
 * rows: the single launch pays at one and two rows; at four rows of a wide
 * (N >= 8192) or deep (K > 4096) product the separate quantize launch costs
 * less than the repeated preparation.
 *   X       bf16 [M, K] in (DEVICE), row stride ldx (multiple of 8, 16-byte
 *           aligned rows)
 *   idx     int32 [k] in (DEVICE): the protected channels, distinct, in
 *           [0, K) (as splice_select_channels writes them); NULL when k == 0
 *   alpha_x float [1] in (DEVICE), > 0 and finite: the frozen activation scale
 *   Wq, Ws, alpha_w, W_S, Y, ldy: as for splice_gemm.
 * Shapes: M <= SPLICE_FUSED_MAX_M; K a multiple of 128 with K <= 16384 (the
 * FP16 copy of X, up to 128 KB, stays in LDS), or K == 0 (Y = 0).
 * Other shapes return SPLICE_ERR_UNSUPPORTED: use the two-call form.
 * No workspace; nothing is allocated; safe inside stream capture. */
#define SPLICE_FUSED_MAX_M 4
int splice_gemm_decode_fused(const uint16_t *X, int64_t ldx, const int32_t *idx,
                             const float *alpha_x, const uint8_t *Wq, const uint8_t *Ws,
                             const float *alpha_w, const uint16_t *W_S, int64_t M, int64_t N,
                             int64_t K, int32_t k, float *Y, int64_t ldy, splice_stream_t stream);

/* ---------------------------------------------------------------------------
 * SpliceGEMM of one set of activation operands against several weight
 * matrices in one launch (Sec. 4.2 Eq. 5 and Sec. 5.1 dual-path execution,
 * per product): the projections that read the same layer input -- q, k and v,
 * or gate and up -- share X's packs, alpha_x and X_S, since the protected
 * channels S are chosen from that input's statistics.  Each segment has its
 * own weight packs, alpha_w, W_S and output.
 *   Xq, Xs, alpha_x, X_S, M, K, k: as for splice_gemm.
 *   segs   HOST array of nseg (1 .. SPLICE_SEG_MAX) entries; in each, Wq, Ws,
 *          alpha_w, W_S, Y and ldy are as splice_gemm's for a product of
 *          width N (N >= 0; 0 skips the segment).
 *   path   as for splice_gemm; the kernel configuration is chosen for M and
 *          the sum of the widths, as one call of that width would choose it.
 * Each segment's Y equals splice_gemm's for that segment alone bit for bit
 * whenever the call alone would make the same plan (splice_gemm_plan against
 * splice_multi_plan: the same path, kernel and K split) -- for the Qwen3-8B
 * q/k/v and gate/up widths it does at M <= 64 and from M = 1024 on -- and
 * within the GEMM tolerance otherwise.  Errors as splice_gemm, checked per segment before
 * anything is launched.
 *   ws, ws_bytes  as for splice_gemm, sized by splice_multi_workspace_size
 *          (the output tiles are counted segment by segment). */
#define SPLICE_SEG_MAX 8
typedef struct {
    const uint8_t *Wq, *Ws;
    const float *alpha_w;
    const uint16_t *W_S;
    int64_t N;
    float *Y;
    int64_t ldy;
} splice_weight_seg;

int splice_gemm_multi(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint16_t *X_S,
                      int64_t M, int64_t K, int32_t k, const splice_weight_seg *segs, int32_t nseg,
                      void *ws, size_t ws_bytes, int path, splice_stream_t stream);

/* splice_gemm_decode_fused over column segments: the bf16 rows X (M <=
 * SPLICE_FUSED_MAX_M), idx and alpha_x as for splice_gemm_decode_fused,
 * shared; segs a HOST array of nseg (1 .. SPLICE_SEG_MAX) weight segments as
 * for splice_gemm_multi.  One launch prepares X in every workgroup and
 * multiplies it by the workgroup's segment.  Each segment's Y equals
 * splice_gemm_decode_fused's for that segment alone, bit for bit: the
 * combined width only decides how many columns a workgroup takes (48 for wide
 * products at two or more rows), never a column's arithmetic.  Errors as
 * splice_gemm_decode_fused, per segment. */
int splice_gemm_decode_fused_multi(const uint16_t *X, int64_t ldx, const int32_t *idx,
                                   const float *alpha_x, int64_t M, int64_t K, int32_t k,
                                   const splice_weight_seg *segs, int32_t nseg, splice_stream_t stream);

/* Workspace bytes splice_gemm / nvfp4_gemm need for this shape, enough for
 * whichever path the call takes (k is part of the contract but does not
 * change the size). */
size_t splice_workspace_size(int64_t M, int64_t N, int64_t K, int32_t k);

/* Workspace bytes splice_gemm_multi needs for these segments (HOST array, as
 * passed to it), enough for whichever path the call takes. */
size_t splice_multi_workspace_size(int64_t M, int64_t K, int32_t k, const splice_weight_seg *segs,
                                   int32_t nseg);

/* Diagnostic: the launch a splice_gemm / nvfp4_gemm call (splice_gemm_plan)
 * or a splice_gemm_multi call (splice_multi_plan) of this shape and path
 * makes, written to plan[0..5): the path taken (1 decode, 2 prefill), a
 * kernel number (0 for every prefill tile size: they sum K in the same
 * order), the output tile of one workgroup (rows, columns) and the number of
 * K ranges the tile's sum is split into.  Two calls with the same M and K
 * whose plans agree in path, kernel number and K ranges run the same
 * arithmetic on every output, so they give the same bits.  Returns SPLICE_ERR_INVALID_ARG for a bad shape,
 * path or pointer; computes nothing on the GPU. */
int splice_gemm_plan(int64_t M, int64_t N, int64_t K, int path, int32_t *plan);
int splice_multi_plan(int64_t M, int64_t K, const splice_weight_seg *segs, int32_t nseg, int path,
                      int32_t *plan);

/* ---------------------------------------------------------------------------
 * Grouped SpliceGEMM: G independent problems sharing N, K and k (experts of
 * an MoE layer, each with its own S, alphas and token count M; the paper's
 * Nemotron3 Up/Down projections, Sec. 6.3).  groups is a HOST array; each
 * entry's pointers are device pointers laid out as for splice_gemm, with
 * ldy = N.  Groups with M == 0 are skipped.  All groups run on the 128x128
 * matrix-core tile of the prefill path, one launch per 32 groups.
 * ws: splice_grouped_workspace_size(groups, G, N, K, k) bytes (currently 0). */
typedef struct {
    const uint8_t *Xq, *Xs;
    const float *alpha_x;
    const uint16_t *X_S;
    const uint8_t *Wq, *Ws;
    const float *alpha_w;
    const uint16_t *W_S;
    int64_t M;
    float *Y;
} splice_group;

int splice_gemm_grouped(const splice_group *groups, int32_t G, int64_t N, int64_t K, int32_t k,
                        void *ws, size_t ws_bytes, splice_stream_t stream);
size_t splice_grouped_workspace_size(const splice_group *groups, int32_t G, int64_t N,
                                     int64_t K, int32_t k);

/* ---------------------------------------------------------------------------
 * TIM-aware sequence filtering (Sec. 4.1 dual-gate mechanism, Eq. 3-4; the
 * paper's settings, Sec. 6.1: tau = 1e-4, K1 = 0.01 x response length,
 * K2 = 5).  For each of B sequences:
 *   logp   float [B, ldl] (DEVICE): training-policy log-probabilities of the
 *          sampled tokens; tokens t >= len[i] are padding and never read.
 *   len    int32 [B] (DEVICE): response lengths; values outside [0, ldl] are
 *          clamped to it.
 *   A token is a tail token when logp <= log_tau (pi_train <= tau).
 *   G1 = tail tokens, G2 = longest run of consecutive tail tokens; the
 *   sequence is kept when G1 * k1_den < k1_num * len (K1 = k1_num/k1_den x
 *   len, exact) and G2 < k2.  An empty response has G1 = 0 = K1 and is
 *   therefore dropped, as Eq. 3 reads.
 *   keep uint8 [B], g1 / g2 int32 [B] out (DEVICE, each may be NULL).
 *   adv    float [B, adv_cols] in/out (DEVICE, row stride lda >= adv_cols, may
 *          be NULL when adv_cols == 0): the rows of dropped sequences are set
 *          to +0, the rest are untouched (Eq. 4; the caller keeps the loss
 *          denominator G).
 * B, ldl, k1_num and k1_den up to 2^31 - 1.  No workspace. */
int splice_tim_filter(const float *logp, int64_t B, int64_t ldl, const int32_t *len, float log_tau,
                      int64_t k1_num, int64_t k1_den, int64_t k2, uint8_t *keep, int32_t *g1,
                      int32_t *g2, float *adv, int64_t adv_cols, int64_t lda,
                      splice_stream_t stream);

/* ---------------------------------------------------------------------------
 * Measurement aid, not part of the SpliceGEMM path: `workgroups` workgroups
 * of 4 waves each issue 4 * iters independent v_mfma_f32_32x32x16_f16 (the
 * prefill tile's instruction) on register operands, 32*32*16*2 flops each;
 * timing the call gives the FP16 matrix-core rate the GPU sustains at its
 * clock under that load.  sink: float [workgroups * 4] out (DEVICE).
 * 2 * (number of CUs) workgroups put two waves on every SIMD. */
int splice_probe_mfma_f16(int64_t iters, int64_t workgroups, float *sink, splice_stream_t stream);

/* Measurement aid, not part of the SpliceGEMM path: a pure streaming read of
 * `bytes` bytes at src (DEVICE, 16-byte aligned, bytes a multiple of 16) by
 * `workgroups` workgroups of 256 threads, each thread with four 16-byte loads
 * in flight per round.  Timing it gives the rate at which this GPU streams a
 * buffer of that size -- the ceiling for a weight-streaming decode call that
 * reads as many bytes.  sink: uint32 [workgroups * 4] out (DEVICE), one
 * folded word per wave. */
int splice_probe_stream_read(const void *src, int64_t bytes, int64_t workgroups, uint32_t *sink,
                             splice_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLICE_H */
