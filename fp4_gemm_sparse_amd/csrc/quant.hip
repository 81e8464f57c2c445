// quant.hip -- channel statistics, top-k channel selection, the FP32 tensor
// scale and the NVFP4 quantize/pack/gather kernel of SpliceGEMM
// (FourSight, arXiv 2611.04887v1: Sec. 4.2 selection, Sec. 5.1 data
// preparation, Sec. 5.2 running channel moments, App. 9.3.1 Eq. 9).
//
// Every floating-point decision here is exact: statistics run in fp64 with
// one IEEE rounding per operation in a fixed order (no contraction), rounding
// decisions of the quantizer compare bf16 inputs against exactly computed
// thresholds.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace splice {

__device__ __forceinline__ float bf16_bits_to_f32(unsigned b) { return __uint_as_float(b << 16); }

// ===========================================================================
// Channel statistics: Welford over 64-row tiles, tiles folded left to right
// with the pairwise update of Chan, Golub & LeVeque, then merged into the
// running moments.  One workgroup owns 64 channels (one per lane); its four
// waves take tiles round-robin and park their tile moments in LDS, and wave 0
// folds them in tile order, so the result does not depend on scheduling.
// ===========================================================================
constexpr int ST_TILE = 64;
constexpr int ST_GROUP = 16;   // tiles parked in LDS per fold round

struct Moments { double n, mean, m2; };

__device__ __forceinline__ Moments chan_merge(Moments a, Moments b)
{
    if (b.n == 0.0) return a;
    if (a.n == 0.0) return b;
    Moments r;
    double n = a.n + b.n;
    double d = b.mean - a.mean;
    r.n = n;
    r.mean = a.mean + d * (b.n / n);
    r.m2 = a.m2 + b.m2 + (d * d) * (a.n * b.n / n);
    return r;
}

__global__ __launch_bounds__(256) void stats_kernel(const uint16_t *__restrict__ X, int64_t T,
                                                    int64_t K, int64_t ldx, int64_t count_prev,
                                                    double *mean, double *m2, float *absmax)
{
    __shared__ double s_mean[ST_GROUP][WAVE];
    __shared__ double s_m2[ST_GROUP][WAVE];
    __shared__ double s_n[ST_GROUP];
    __shared__ float s_amax[4][WAVE];
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    const int64_t j = (int64_t)blockIdx.x * WAVE + lane;
    const bool valid = j < K;
    Moments acc = {0.0, 0.0, 0.0};
    float amax = 0.0f;
    const int64_t ntiles = (T + ST_TILE - 1) / ST_TILE;
    for (int64_t g0 = 0; g0 < ntiles; g0 += ST_GROUP) {
        const int gt = (int)min((int64_t)ST_GROUP, ntiles - g0);
        for (int t = wave; t < gt; t += 4) {
            const int64_t r0 = (g0 + t) * ST_TILE;
            const int64_t r1 = min(r0 + ST_TILE, T);
            double n = 0.0, mu = 0.0, M2 = 0.0;
            if (valid) {
                for (int64_t r = r0; r < r1; r++) {
                    const float xf = bf16_bits_to_f32(X[r * ldx + j]);
                    const double x = (double)xf;
                    n += 1.0;
                    const double d = x - mu;
                    mu += d / n;
                    M2 += d * (x - mu);
                    amax = fmaxf(amax, fabsf(xf));
                }
            }
            s_mean[t][lane] = mu;
            s_m2[t][lane] = M2;
            if (lane == 0) s_n[t] = (double)(r1 - r0);
        }
        __syncthreads();
        if (wave == 0) {
            for (int t = 0; t < gt; t++) {
                Moments tile = {s_n[t], s_mean[t][lane], s_m2[t][lane]};
                acc = chan_merge(acc, tile);
            }
        }
        __syncthreads();
    }
    s_amax[wave][lane] = amax;
    __syncthreads();
    if (wave == 0 && valid) {
        float a = fmaxf(fmaxf(s_amax[0][lane], s_amax[1][lane]), fmaxf(s_amax[2][lane], s_amax[3][lane]));
        Moments run = {0.0, 0.0, 0.0};
        float prev = 0.0f;
        if (count_prev > 0) {
            run.n = (double)count_prev;
            run.mean = mean[j];
            run.m2 = m2[j];
            prev = absmax[j];
        }
        run = chan_merge(run, acc);
        mean[j] = run.mean;
        m2[j] = run.m2;
        absmax[j] = fmaxf(a, prev);
    }
}

hipError_t launch_stats(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int64_t count_prev,
                        double *mean, double *m2, float *absmax, hipStream_t s)
{
    if (K == 0) return hipSuccess;
    dim3 grid((unsigned)((K + WAVE - 1) / WAVE));
    hipLaunchKernelGGL(stats_kernel, grid, dim3(256), 0, s, X, T, K, ldx, count_prev, mean, m2,
                       absmax);
    return hipGetLastError();
}

// ===========================================================================
// Top-k selection: the k channels with the largest M2, ties to the lower
// index, written in ascending channel order; plus the frozen activation scale
// (largest absmax over the channels left unprotected) / 2688.
// One workgroup: an 8-pass radix select over a total-order key of the fp64
// M2 finds the k-th largest key and how many of the keys equal to it are
// taken (the lowest-indexed ones); two scans then compact the selection.
// ===========================================================================
constexpr int SEL_THREADS = 1024;

__device__ __forceinline__ uint64_t order_key(double v)
{
    uint64_t u = (uint64_t)__double_as_longlong(v);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// exclusive scan of one int64 per thread over the workgroup
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *buf)
{
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < SEL_THREADS; off <<= 1) {
        int64_t t = (tid >= off) ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += t;
        __syncthreads();
    }
    int64_t incl = buf[tid];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const double *__restrict__ m2,
                                                             const float *__restrict__ absmax,
                                                             int64_t K, int32_t k, int32_t *idx,
                                                             float *alpha_x)
{
    __shared__ unsigned hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ int64_t s_need;
    __shared__ int64_t s_buf[SEL_THREADS];
    __shared__ float s_max[SEL_THREADS / WAVE];
    const int tid = threadIdx.x;
    const int64_t per = (K + SEL_THREADS - 1) / SEL_THREADS;
    const int64_t c0 = min(K, (int64_t)tid * per), c1 = min(K, c0 + per);

    uint64_t thr = 0;       // key of the k-th largest channel
    int64_t need = 0;       // how many channels with key == thr are taken
    if (k > 0) {
        uint64_t prefix = 0, pmask = 0;
        int64_t remaining = k;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
            __syncthreads();
            for (int64_t j = c0; j < c1; j++) {
                uint64_t key = order_key(m2[j]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                int64_t cum = 0;
                int d = 255;
                for (; d > 0; d--) {
                    if (cum + (int64_t)hist[d] >= remaining) break;
                    cum += hist[d];
                }
                s_prefix = prefix | ((uint64_t)d << shift);
                s_need = remaining - cum;
            }
            __syncthreads();
            prefix = s_prefix;
            remaining = s_need;
            pmask |= (uint64_t)255 << shift;
            __syncthreads();
        }
        thr = prefix;
        need = remaining;
    }

    int64_t my_eq = 0;
    if (k > 0)
        for (int64_t j = c0; j < c1; j++) my_eq += (order_key(m2[j]) == thr);
    const int64_t eq_before = block_exclusive_scan(my_eq, s_buf);

    int64_t my_sel = 0;
    {
        int64_t e = eq_before;
        if (k > 0)
            for (int64_t j = c0; j < c1; j++) {
                const uint64_t key = order_key(m2[j]);
                const bool eq = key == thr;
                my_sel += (key > thr) || (eq && e < need);
                e += eq;
            }
    }
    int64_t p = block_exclusive_scan(my_sel, s_buf);

    float am = 0.0f;
    {
        int64_t e = eq_before;
        for (int64_t j = c0; j < c1; j++) {
            bool sel = false;
            if (k > 0) {
                const uint64_t key = order_key(m2[j]);
                const bool eq = key == thr;
                sel = (key > thr) || (eq && e < need);
                e += eq;
            }
            if (sel) idx[p++] = (int32_t)j;
            else am = fmaxf(am, absmax[j]);
        }
    }
    if (alpha_x) {
        for (int off = WAVE / 2; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
        if (tid % WAVE == 0) s_max[tid / WAVE] = am;
        __syncthreads();
        if (tid == 0) {
            float a = 0.0f;
            for (int w = 0; w < SEL_THREADS / WAVE; w++) a = fmaxf(a, s_max[w]);
            *alpha_x = (a == 0.0f) ? 1.0f : __fdiv_rn(a, 2688.0f);
        }
    }
}

hipError_t launch_select(const double *m2, const float *absmax, int64_t K, int32_t k, int32_t *idx,
                         float *alpha_x, hipStream_t s)
{
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(SEL_THREADS), 0, s, m2, absmax, K, k, idx,
                       alpha_x);
    return hipGetLastError();
}

// ===========================================================================
// Protected-channel bitmask in LDS (bit j of the mask = channel j is in S).
// ===========================================================================
constexpr int MAX_K = 65536;

__device__ __forceinline__ void build_mask(uint32_t *smask, int64_t K, const int32_t *idx,
                                           int32_t k)
{
    const int words = (int)((K + 31) / 32);
    for (int i = threadIdx.x; i < words; i += blockDim.x) smask[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        const int c = idx[i];
        if (c >= 0 && c < K) atomicOr(&smask[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
}

__device__ __forceinline__ unsigned block_mask16(const uint32_t *smask, int64_t b)
{
    return (smask[b >> 1] >> ((b & 1) * 16)) & 0xFFFFu;
}

// ===========================================================================
// Masked amax -> alpha = fp32(amax / 2688), 1 when amax is 0.
// ===========================================================================
constexpr int AMAX_GRID = 1024;
size_t alpha_ws_bytes() { return AMAX_GRID * sizeof(unsigned); }

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t *__restrict__ A, int64_t R,
                                                   int64_t K, int64_t lda,
                                                   const int32_t *__restrict__ idx, int32_t k,
                                                   unsigned *partial)
{
    __shared__ uint32_t smask[MAX_K / 32];
    __shared__ unsigned s_red[4];
    if (k > 0) build_mask(smask, K, idx, k);
    const int64_t nb = K / NVFP4_BLOCK;
    const int64_t total = R * nb;
    unsigned amax = 0;
    for (int64_t task = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; task < total;
         task += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = task / nb, b = task - r * nb;
        const u32x4 *p = reinterpret_cast<const u32x4 *>(A + r * lda + b * NVFP4_BLOCK);
        const u32x4 v0 = p[0], v1 = p[1];
        const unsigned m = (k > 0) ? block_mask16(smask, b) : 0u;
        const unsigned w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int t = 0; t < 16; t++) {
            const unsigned x = (w[t >> 1] >> ((t & 1) * 16)) & 0x7FFFu;
            amax = ((m >> t) & 1u) ? amax : max(amax, x);
        }
    }
    for (int off = WAVE / 2; off > 0; off >>= 1) amax = max(amax, (unsigned)__shfl_xor((int)amax, off));
    if (threadIdx.x % WAVE == 0) s_red[threadIdx.x / WAVE] = amax;
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.x] = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
}

__global__ __launch_bounds__(256) void alpha_final_kernel(const unsigned *partial, int n,
                                                          float *alpha)
{
    __shared__ unsigned s_red[4];
    unsigned a = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) a = max(a, partial[i]);
    for (int off = WAVE / 2; off > 0; off >>= 1) a = max(a, (unsigned)__shfl_xor((int)a, off));
    if (threadIdx.x % WAVE == 0) s_red[threadIdx.x / WAVE] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        a = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
        *alpha = (a == 0u) ? 1.0f : __fdiv_rn(bf16_bits_to_f32(a), 2688.0f);
    }
}

hipError_t launch_alpha(const uint16_t *A, int64_t R, int64_t K, int64_t lda, const int32_t *idx,
                        int32_t k, float *alpha, void *ws, hipStream_t s)
{
    unsigned *partial = static_cast<unsigned *>(ws);
    hipLaunchKernelGGL(amax_kernel, dim3(AMAX_GRID), dim3(256), 0, s, A, R, K, lda, idx, k,
                       partial);
    hipLaunchKernelGGL(alpha_final_kernel, dim3(1), dim3(256), 0, s, partial, AMAX_GRID, alpha);
    return hipGetLastError();
}

// ===========================================================================
// NVFP4 quantization of the masked residual, plus the side-buffer gather.
// One thread per 16-element block: two 16-byte loads, the block amax with the
// protected lanes read as +0, the E4M3 scale, sixteen E2M1 codes, one 8-byte
// store of codes, one scale byte, and the protected values copied to their
// slot of the compact side buffer.
//
// Exact decisions:
//  - scale: v = a_b / (6 alpha) in fp64 (6 alpha exact; the quotient of an
//    8-bit by a 26-bit operand is never within 2^-53 of an E4M3 rounding
//    midpoint unless it equals it), then round-to-nearest-even onto E4M3FN
//    with saturation at 448;
//  - codes: the seven midpoints m_i of the E2M1 grid times s_b*alpha are exact
//    in fp64 (3 x 4 x 24 bits); each is turned into the fp32 bit pattern the
//    bf16 inputs are compared against (rounded down when not representable,
//    one step lower for the midpoints whose ties round up to the even code),
//    so that code = number of patterns below |x|'s pattern, exactly.
// ===========================================================================

// Round v >= 0 to E4M3FN, nearest, ties to even mantissa, saturating at 448.
__device__ __forceinline__ unsigned e4m3_rne_sat(double v)
{
    if (v >= 448.0) return 0x7Eu;
    if (v < 0.015625) return (unsigned)rint(v * 512.0);          // subnormals: m * 2^-9, m <= 8
    const int e = ilogb(v);                                       // -6 .. 8
    const int n = (int)rint(ldexp(v, 3 - e));                     // 8 .. 16
    return (unsigned)(((e + 7) << 3) + n - 8);
}

__device__ __forceinline__ double e4m3_value(unsigned b)
{
    const int e = (b >> 3) & 15, m = b & 7;
    return e ? ldexp(1.0 + (double)m * 0.125, e - 7) : ldexp((double)m, -9);
}

// fp32 bit pattern of the largest float <= t (t > 0), and whether it equals t.
__device__ __forceinline__ unsigned f32_bits_round_down(double t, bool &exact)
{
    const uint64_t u = (uint64_t)__double_as_longlong(t);
    const int ed = (int)((u >> 52) & 0x7FF);
    const uint64_t mant = u & 0xFFFFFFFFFFFFFull;
    if (ed - 1023 >= 128) { exact = false; return 0x7F7FFFFFu; }  // beyond FLT_MAX
    if (ed - 1023 >= -126) {                                       // fp32 normal range
        exact = (mant & ((1ull << 29) - 1)) == 0;
        return ((unsigned)(ed - 1023 + 127) << 23) | (unsigned)(mant >> 29);
    }
    const double q = ldexp(t, 149);                                // fp32 subnormal units
    const double f = floor(q);
    exact = (f == q);
    return (unsigned)f;
}

__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t *__restrict__ A, int64_t R, int64_t K, int64_t lda,
    const int32_t *__restrict__ idx, int32_t k, const float *__restrict__ alpha_p,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint16_t *__restrict__ side)
{
    __shared__ uint32_t smask[MAX_K / 32];
    __shared__ uint32_t spre[MAX_K / NVFP4_BLOCK];
    __shared__ int64_t s_scan[256];
    const int64_t nb = K / NVFP4_BLOCK;
    if (k > 0) {
        build_mask(smask, K, idx, k);
        // exclusive prefix (over blocks) of the number of protected channels
        const int64_t cpt = (nb + 255) / 256;
        const int64_t b0 = min(nb, (int64_t)threadIdx.x * cpt), b1 = min(nb, b0 + cpt);
        int64_t local = 0;
        for (int64_t b = b0; b < b1; b++) local += __popc(block_mask16(smask, b));
        s_scan[threadIdx.x] = local;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            int64_t t = (threadIdx.x >= (unsigned)off) ? s_scan[threadIdx.x - off] : 0;
            __syncthreads();
            s_scan[threadIdx.x] += t;
            __syncthreads();
        }
        int64_t base = s_scan[threadIdx.x] - local;
        for (int64_t b = b0; b < b1; b++) {
            spre[b] = (uint32_t)base;
            base += __popc(block_mask16(smask, b));
        }
        __syncthreads();
    }
    const double alpha = (double)*alpha_p;
    const double six_alpha = 6.0 * alpha;
    const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    const int64_t total = R * nb;
    for (int64_t task = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; task < total;
         task += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = task / nb, b = task - r * nb;
        const uint16_t *src = A + r * lda + b * NVFP4_BLOCK;
        const u32x4 v0 = reinterpret_cast<const u32x4 *>(src)[0];
        const u32x4 v1 = reinterpret_cast<const u32x4 *>(src)[1];
        const unsigned w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const unsigned m = (k > 0) ? block_mask16(smask, b) : 0u;
        unsigned amax = 0;
#pragma unroll
        for (int t = 0; t < 16; t++) {
            const unsigned x = (w[t >> 1] >> ((t & 1) * 16)) & 0x7FFFu;
            amax = ((m >> t) & 1u) ? amax : max(amax, x);
        }
        const unsigned sc = e4m3_rne_sat((double)bf16_bits_to_f32(amax) / six_alpha);
        unsigned key[7];
        if (sc != 0) {
            const double phys = e4m3_value(sc) * alpha;               // exact
#pragma unroll
            for (int i = 0; i < 7; i++) {
                bool exact;
                unsigned kb = f32_bits_round_down(mids[i] * phys, exact);
                key[i] = (exact && (i & 1)) ? kb - 1u : kb;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 7; i++) key[i] = 0xFFFFFFFFu;          // every code 0
        }
        unsigned lo = 0, hi = 0;
#pragma unroll
        for (int t = 0; t < 16; t++) {
            const unsigned raw = (w[t >> 1] >> ((t & 1) * 16)) & 0xFFFFu;
            const bool prot = (m >> t) & 1u;
            const unsigned xk = prot ? 0u : (raw & 0x7FFFu) << 16;
            unsigned c = 0;
#pragma unroll
            for (int i = 0; i < 7; i++) c += (xk > key[i]) ? 1u : 0u;
            const unsigned nib = (prot ? 0u : ((raw >> 15) << 3)) | c;
            if (t < 8) lo |= nib << (4 * t);
            else hi |= nib << (4 * (t - 8));
        }
        *reinterpret_cast<u32x2 *>(codes + r * (K / 2) + b * 8) = u32x2{lo, hi};
        scales[r * nb + b] = (uint8_t)sc;
        if (m) {
            const unsigned base = spre[b];
#pragma unroll
            for (int t = 0; t < 16; t++)
                if ((m >> t) & 1u)
                    side[r * (int64_t)k + base + __popc(m & ((1u << t) - 1u))] =
                        (uint16_t)((w[t >> 1] >> ((t & 1) * 16)) & 0xFFFFu);
        }
    }
}

hipError_t launch_quantize(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                           const int32_t *idx, int32_t k, const float *alpha, uint8_t *codes,
                           uint8_t *scales, uint16_t *side, hipStream_t s)
{
    const int64_t total = R * (K / NVFP4_BLOCK);
    if (total == 0) return hipSuccess;
    const int64_t blocks = min((total + 255) / 256, (int64_t)2048);
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, A, R, K, lda, idx,
                       k, alpha, codes, scales, side);
    return hipGetLastError();
}

}  // namespace splice
