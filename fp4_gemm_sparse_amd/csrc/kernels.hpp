// kernels.hpp -- internal launchers behind the C ABI (not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace splice {

// channel statistics + top-k (+ frozen activation scale)
hipError_t launch_stats(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int64_t count_prev,
                        double *mean, double *m2, float *absmax, hipStream_t s);
// mean == nullptr: rank by M2 (variance); else by m2/count + mean^2
hipError_t launch_select(const double *m2, const double *mean, int64_t count, const float *absmax,
                         int64_t K, int32_t k, int32_t *idx, float *alpha_x, hipStream_t s);

// masked amax -> alpha
size_t alpha_ws_bytes();
hipError_t launch_alpha(const uint16_t *A, int64_t R, int64_t K, int64_t lda, const int32_t *idx,
                        int32_t k, float *alpha, void *ws, hipStream_t s);

// mask + NVFP4 quantize + side gather
hipError_t launch_quantize(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                           const int32_t *idx, int32_t k, const float *alpha, uint8_t *codes,
                           uint8_t *scales, uint16_t *side, hipStream_t s);

// GEMMs
struct GemmArgs {
    const uint8_t *Xq, *Xs;
    const float *alpha_x;
    const uint16_t *X_S;
    const uint8_t *Wq, *Ws;
    const float *alpha_w;
    const uint16_t *W_S;
    int64_t M, N, K;
    int32_t k;
    float *Y;
    int64_t ldy;
    // activation-prep fused decode only: bf16 X [M, K] with row stride ldx and
    // the protected channels idx[0..k); Xq, Xs and X_S are then unused
    const uint16_t *X;
    int64_t ldx;
    const int32_t *idx;
};
enum class Path { Decode, Prefill };
// a K-split launch's workspace: SPLIT_COUNTER_BYTES of arrival counters (one
// word per output tile), then the partial tiles
constexpr size_t SPLIT_COUNTER_BYTES = 1024;
size_t gemm_ws_bytes(Path p, int64_t M, int64_t N, int64_t K);
struct GemmSeg;
size_t gemm_seg_ws_bytes(Path p, int64_t M, int64_t K, const GemmSeg *seg, int nseg);
// {path taken (1 decode, 2 prefill), kernel, tile rows, tile columns, K splits}
// of a call of this shape (seg: the column segments of a multi launch, or null)
void gemm_plan_info(Path p, int64_t M, int64_t N, int64_t K, const GemmSeg *seg, int nseg, int32_t out[5]);
hipError_t launch_gemm(Path p, const GemmArgs &a, void *ws, size_t ws_bytes, hipStream_t s);
// one column segment of a launch that shares the activation operands: its
// own weights, tensor scale, side columns and output of width N
struct GemmSeg {
    const uint8_t *Wq, *Ws;
    const float *alpha_w;
    const uint16_t *W_S;
    float *Y;
    int64_t ldy, N;
};
constexpr int SEG_MAX = 8;
struct SegSpec {
    const GemmSeg *seg;
    int nseg;
};
// the products of a's activation operands (Xq, Xs, alpha_x, X_S, M, K, k)
// with each segment's weights, in one launch (a's weight and output fields
// are ignored); 1 <= nseg <= SEG_MAX
hipError_t launch_gemm_seg(Path p, const GemmArgs &a, const GemmSeg *seg, int nseg, void *ws, hipStream_t s);
// launch_gemm_fused over column segments (a's weight and output fields ignored)
hipError_t launch_gemm_fused_seg(const GemmArgs &a, const GemmSeg *seg, int nseg, hipStream_t s);
// independent products sharing N, K and k (groups[i].N/K/k equal), one launch
// per 32 groups; groups with M == 0 are skipped
hipError_t launch_gemm_grouped(const GemmArgs *groups, int G, hipStream_t s);
// decode GEMM that quantizes X itself (GemmArgs.X/ldx/idx, alpha_x); shapes
// for which fused_decode_ok holds
bool fused_decode_ok(int64_t M, int64_t K);
hipError_t launch_gemm_fused(const GemmArgs &a, hipStream_t s);

// TIM-aware sequence filter (tim.hip)
struct TimArgs {
    const float *logp;
    int64_t B, ldl;
    const int32_t *len;
    float log_tau;
    int64_t k1_num, k1_den, k2;
    uint8_t *keep;
    int32_t *g1, *g2;
    float *adv;
    int64_t adv_cols, lda;
};
hipError_t launch_tim_filter(const TimArgs &a, hipStream_t s);

// measurement aid: `workgroups` x 4 waves, each 4 * iters 32x32x16 FP16 MFMAs
hipError_t launch_mfma_rate(int64_t iters, int64_t workgroups, float *sink, hipStream_t s);
// measurement aid: a pure read of `bytes` (a multiple of 16) by `workgroups`
// x 256 threads; sink receives one word per wave
hipError_t launch_stream_read(const void *src, int64_t bytes, int64_t workgroups, unsigned *sink,
                              hipStream_t s);

}  // namespace splice
