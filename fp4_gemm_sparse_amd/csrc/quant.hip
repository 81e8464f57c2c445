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
#include "nvfp4.hpp"

#pragma clang fp contract(off)

namespace splice {


// ===========================================================================
// Channel statistics: Welford over 64-row tiles, tiles folded left to right
// with the pairwise update of Chan, Golub & LeVeque, then merged into the
// running moments.  One workgroup owns 64 channels (one per lane).  Its eight
// waves each take one tile of a round of eight: a wave issues the loads of
// all 64 rows of its tile (one round trip) before it starts their (serial)
// Welford steps, parks the tile moments
// in LDS, and wave 0 folds the round in tile order, so the result does not
// depend on scheduling.
// ===========================================================================
constexpr int ST_TILE = 64;
constexpr int ST_WAVES = 8;    // tiles per fold round, one per wave
constexpr int ST_BATCH = 64;   // rows loaded ahead of their Welford steps (a whole tile)

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

__global__ __launch_bounds__(ST_WAVES * WAVE) void stats_kernel(
    const uint16_t *__restrict__ X, int64_t T, int64_t K, int64_t ldx, int64_t count_prev,
    double *mean, double *m2, float *absmax)
{
    __shared__ double s_mean[ST_WAVES][WAVE];
    __shared__ double s_m2[ST_WAVES][WAVE];
    __shared__ float s_amax[ST_WAVES][WAVE];
    const int lane = threadIdx.x % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int64_t j = (int64_t)blockIdx.x * WAVE + lane;
    const bool valid = j < K;
    const int64_t jc = valid ? j : K - 1;          // lanes past K read a valid column, unused
    Moments acc = {0.0, 0.0, 0.0};
    float amax = 0.0f;
    const int64_t ntiles = (T + ST_TILE - 1) / ST_TILE;
    for (int64_t g0 = 0; g0 < ntiles; g0 += ST_WAVES) {
        const int gt = (int)min((int64_t)ST_WAVES, ntiles - g0);
        if (wave < gt) {
            const int64_t r0 = (g0 + wave) * ST_TILE;
            const int rows = (int)min((int64_t)ST_TILE, T - r0);
            const uint16_t *p = X + r0 * ldx + jc;
            double n = 0.0, mu = 0.0, M2 = 0.0;
            for (int c = 0; c < rows; c += ST_BATCH) {
                float v[ST_BATCH];
#pragma unroll
                for (int u = 0; u < ST_BATCH; u++)
                    v[u] = bf16_bits_to_f32(p[(int64_t)min(c + u, rows - 1) * ldx]);
#pragma unroll
                for (int u = 0; u < ST_BATCH; u++) {
                    if (c + u < rows) {
                        const double x = (double)v[u];
                        n += 1.0;
                        const double d = x - mu;
                        mu += d / n;
                        M2 += d * (x - mu);
                        amax = fmaxf(amax, fabsf(v[u]));
                    }
                }
            }
            s_mean[wave][lane] = mu;
            s_m2[wave][lane] = M2;
        }
        __syncthreads();
        if (wave == 0) {
            for (int t = 0; t < gt; t++) {
                const double nt = (double)min((int64_t)ST_TILE, T - (g0 + t) * ST_TILE);
                Moments tile = {nt, s_mean[t][lane], s_m2[t][lane]};
                acc = chan_merge(acc, tile);
            }
        }
        __syncthreads();
    }
    s_amax[wave][lane] = amax;
    __syncthreads();
    if (wave == 0 && valid) {
        float a = 0.0f;
        for (int w = 0; w < ST_WAVES; w++) a = fmaxf(a, s_amax[w][lane]);
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
    hipLaunchKernelGGL(stats_kernel, grid, dim3(ST_WAVES * WAVE), 0, s, X, T, K, ldx, count_prev,
                       mean, m2, absmax);
    return hipGetLastError();
}

// ===========================================================================
// Top-k selection: the k channels with the largest M2 (variance), or with
// the largest second moment m2/n + mean^2 (the minimiser of the relaxed error
// bound, FourSight App. Prop. 2 / Cor. 1), ties to the lower index, written in
// ascending channel order; plus the frozen activation scale (largest absmax
// over the channels left unprotected) / 2688.
// One workgroup: an 8-pass radix select over a total-order key of the fp64
// ranking value finds the k-th largest key and how many of the keys equal to
// it are taken (the lowest-indexed ones); two scans then compact the
// selection.
// ===========================================================================
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;

__device__ __forceinline__ uint64_t order_key(double v)
{
    uint64_t u = (uint64_t)__double_as_longlong(v);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive scan of one int64 per thread over the workgroup: a shuffle scan in
// each wave, then a scan of the wave totals.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *wtot)
{
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    int64_t incl = v;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const int64_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == WAVE - 1) wtot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int64_t x = lane < SEL_WAVES ? wtot[lane] : 0;
#pragma unroll
        for (int off = 1; off < SEL_WAVES; off <<= 1) {
            const int64_t t = __shfl_up(x, off);
            if (lane >= off) x += t;
        }
        if (lane < SEL_WAVES) wtot[SEL_WAVES + lane] = x - wtot[lane];
    }
    __syncthreads();
    const int64_t r = wtot[SEL_WAVES + wave] + incl - v;
    __syncthreads();
    return r;
}

// hist[d] += 1 for every active lane: lanes holding the wave's most common
// digits are counted with one atomic per digit (a few rounds), the rest with
// one atomic each.
__device__ __forceinline__ void hist_add(unsigned *hist, unsigned d, bool active)
{
    const int lane = threadIdx.x % WAVE;
    for (int round = 0; round < 4; round++) {
        const uint64_t act = __ballot(active);
        if (act == 0) return;
        const int lead = __builtin_ctzll(act);
        const unsigned dl = (unsigned)__shfl((int)d, lead);
        const bool same = active && d == dl;
        const uint64_t m = __ballot(same);
        if (lane == lead) atomicAdd(&hist[dl], (unsigned)__popcll(m));
        if (same) active = false;
    }
    if (active) atomicAdd(&hist[d], 1u);
}

// Ranking value of channel j: M2, or with mean != nullptr the second moment
// m2/n + mean^2 (one IEEE rounding per operation; 0 before any row).
struct RankValue {
    const double *m2, *mean;
    double n;
    __device__ __forceinline__ double operator()(int64_t j) const
    {
        if (!mean) return m2[j];
        if (n == 0.0) return 0.0;
        const double v = m2[j] / n;
        const double mu2 = mean[j] * mean[j];
        return v + mu2;
    }
};

// The order keys of a thread's channels c0 .. c1-1: held in registers when
// PER > 0 (at most PER per thread), recomputed otherwise.
template <int PER>
struct KeySource {
    uint64_t reg[PER > 0 ? PER : 1];
    RankValue val;
    int64_t c0, c1;
    __device__ __forceinline__ void init(const RankValue &v, int64_t a, int64_t b)
    {
        val = v;
        c0 = a;
        c1 = b;
        if (PER > 0) {
#pragma unroll
            for (int i = 0; i < (PER > 0 ? PER : 1); i++) reg[i] = (c0 + i < c1) ? order_key(val(c0 + i)) : 0;
        }
    }
    __device__ __forceinline__ uint64_t operator()(int i) const
    {
        if (PER > 0) {
            uint64_t v = 0;
#pragma unroll
            for (int q = 0; q < (PER > 0 ? PER : 1); q++) v = (q == i) ? reg[q] : v;
            return v;
        }
        return order_key(val(c0 + i));
    }
};

template <int PER>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(RankValue rv,
                                                             const float *__restrict__ absmax,
                                                             int64_t K, int32_t k, int32_t *idx,
                                                             float *alpha_x)
{
    __shared__ unsigned hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ int64_t s_need, s_bin;
    __shared__ int64_t s_wtot[2 * SEL_WAVES];
    __shared__ float s_max[SEL_WAVES];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int per = (int)((K + SEL_THREADS - 1) / SEL_THREADS);
    const int64_t c0 = min(K, (int64_t)tid * per), c1 = min(K, c0 + per);
    const int n = (int)(c1 - c0);
    KeySource<PER> keys;
    keys.init(rv, c0, c1);

    uint64_t thr = 0;       // key bits (under pmask) of the k-th largest channel
    uint64_t pmask = 0;     // the key bits decided so far
    int64_t need = 0;       // how many channels whose key matches thr under pmask are taken
    if (k > 0) {
        uint64_t prefix = 0;
        int64_t remaining = k;
        // radix passes from the top byte down; they stop early once the bin
        // that holds the k-th key holds exactly the keys still needed (all
        // of them are then taken, whatever their lower bits)
        for (int shift = 56; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int i = 0; i < per; i++) {                   // same trip count in every lane
                const bool in = i < n;
                const uint64_t key = in ? keys(i) : 0;
                hist_add(hist, (unsigned)(key >> shift) & 255u, in && (key & pmask) == prefix);
            }
            __syncthreads();
            if (tid < WAVE) {
                // lane l covers digits 255-4l .. 252-4l; find the digit d where the
                // count of keys with a larger digit first reaches `remaining`
                unsigned h[4], sum = 0;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    h[q] = hist[255 - 4 * lane - q];
                    sum += h[q];
                }
                unsigned incl = sum;
#pragma unroll
                for (int off = 1; off < WAVE; off <<= 1) {
                    const unsigned t = __shfl_up(incl, off);
                    if (lane >= off) incl += t;
                }
                int64_t before = (int64_t)(incl - sum);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if (before < remaining && before + (int64_t)h[q] >= remaining) {
                        s_prefix = prefix | ((uint64_t)(255 - 4 * lane - q) << shift);
                        s_need = remaining - before;
                        s_bin = (int64_t)h[q];
                    }
                    before += h[q];
                }
            }
            __syncthreads();
            prefix = s_prefix;
            remaining = s_need;
            const bool whole_bin = s_bin == remaining;
            pmask |= (uint64_t)255 << shift;
            __syncthreads();
            if (whole_bin) break;                      // uniform: read from LDS by every thread
        }
        thr = prefix;
        need = remaining;
    }

    int64_t my_eq = 0;
    if (k > 0)
        for (int i = 0; i < n; i++) my_eq += ((keys(i) & pmask) == thr);
    const int64_t eq_before = block_exclusive_scan(my_eq, s_wtot);

    int64_t my_sel = 0;
    {
        int64_t e = eq_before;
        if (k > 0)
            for (int i = 0; i < n; i++) {
                const uint64_t key = keys(i) & pmask;
                const bool eq = key == thr;
                my_sel += (key > thr) || (eq && e < need);
                e += eq;
            }
    }
    int64_t p = block_exclusive_scan(my_sel, s_wtot);

    float am = 0.0f;
    {
        int64_t e = eq_before;
        for (int i = 0; i < n; i++) {
            bool sel = false;
            if (k > 0) {
                const uint64_t key = keys(i) & pmask;
                const bool eq = key == thr;
                sel = (key > thr) || (eq && e < need);
                e += eq;
            }
            if (sel) idx[p++] = (int32_t)(c0 + i);
            else am = fmaxf(am, absmax[c0 + i]);
        }
    }
    if (alpha_x) {
        for (int off = WAVE / 2; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
        if (lane == 0) s_max[tid / WAVE] = am;
        __syncthreads();
        if (tid == 0) {
            float a = 0.0f;
            for (int w = 0; w < SEL_WAVES; w++) a = fmaxf(a, s_max[w]);
            *alpha_x = (a == 0.0f) ? 1.0f : __fdiv_rn(a, 2688.0f);
        }
    }
}

hipError_t launch_select(const double *m2, const double *mean, int64_t count, const float *absmax,
                         int64_t K, int32_t k, int32_t *idx, float *alpha_x, hipStream_t s)
{
    const RankValue rv{m2, mean, (double)count};
    const int64_t per = (K + SEL_THREADS - 1) / SEL_THREADS;
    if (per <= 4)
        hipLaunchKernelGGL(select_kernel<4>, dim3(1), dim3(SEL_THREADS), 0, s, rv, absmax, K, k,
                           idx, alpha_x);
    else if (per <= 16)
        hipLaunchKernelGGL(select_kernel<16>, dim3(1), dim3(SEL_THREADS), 0, s, rv, absmax, K, k,
                           idx, alpha_x);
    else
        hipLaunchKernelGGL(select_kernel<0>, dim3(1), dim3(SEL_THREADS), 0, s, rv, absmax, K, k,
                           idx, alpha_x);
    return hipGetLastError();
}

// Walks the (row, block) pairs of one thread: rows blockIdx.x, +gridDim.x, ...
// and blocks threadIdx.x, +ROW_THREADS, ... of each row.  Loops take U pairs
// per step and issue all their loads before using any (rows past the end are
// clamped to the last row, so every load is in bounds; their results are
// discarded).
constexpr int ROW_THREADS = 256;

struct RowBlockWalk {
    int64_t r;
    int b;
    __device__ __forceinline__ void next(int nb)
    {
        b += ROW_THREADS;
        if (b >= nb) {
            b = threadIdx.x;
            r += gridDim.x;
        }
    }
};

// ===========================================================================
// Masked amax -> alpha = fp32(amax / 2688), 1 when amax is 0.
// ===========================================================================
constexpr int AMAX_GRID = 2048;
size_t alpha_ws_bytes() { return AMAX_GRID * sizeof(unsigned); }

// One workgroup per row (grid-stride over rows), one thread per block.
template <bool PROT>
__global__ __launch_bounds__(ROW_THREADS) void amax_kernel(const uint16_t *__restrict__ A, int64_t R,
                                                           int64_t K, int64_t lda,
                                                           const int32_t *__restrict__ idx,
                                                           int32_t k, unsigned *partial)
{
    __shared__ uint32_t smask[MAX_K / 32];
    __shared__ unsigned s_red[ROW_THREADS / WAVE];
    if (PROT) build_mask(smask, K, idx, k);
    const int nb = (int)(K / NVFP4_BLOCK);
    unsigned amax = 0;
    constexpr int U = 4;
    RowBlockWalk it{(int64_t)blockIdx.x, (int)threadIdx.x};
    if (it.b < nb)
        while (it.r < R) {
            RowBlockWalk w[U];
            Block16 x[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                w[u] = it;
                it.next(nb);
                x[u] = load_block(A + min(w[u].r, R - 1) * lda + w[u].b * NVFP4_BLOCK);
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (w[u].r < R) {
                    if (PROT) {
                        const unsigned m = block_mask16(smask, w[u].b);
                        if (m) clear_protected(x[u], m);
                    }
                    amax = max(amax, block_amax_bits(x[u]));
                }
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
    const int grid = (int)max((int64_t)1, min(R, (int64_t)AMAX_GRID));
    if (k > 0)
        hipLaunchKernelGGL(amax_kernel<true>, dim3(grid), dim3(ROW_THREADS), 0, s, A, R, K, lda,
                           idx, k, partial);
    else
        hipLaunchKernelGGL(amax_kernel<false>, dim3(grid), dim3(ROW_THREADS), 0, s, A, R, K, lda,
                           idx, k, partial);
    hipLaunchKernelGGL(alpha_final_kernel, dim3(1), dim3(256), 0, s, partial, grid, alpha);
    return hipGetLastError();
}

template <bool PROT>
__global__ __launch_bounds__(ROW_THREADS) void quantize_kernel(
    const uint16_t *__restrict__ A, int64_t R, int64_t K, int64_t lda,
    const int32_t *__restrict__ idx, int32_t k, const float *__restrict__ alpha_p,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint16_t *__restrict__ side)
{
    __shared__ uint32_t smask[MAX_K / 32];
    if (PROT) build_mask(smask, K, idx, k);
    const TensorScale ts = tensor_scale(*alpha_p);
    const int nb = (int)(K / NVFP4_BLOCK);
    for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
        const uint16_t *row = A + r * lda;
        uint8_t *crow = codes + r * (K / 2);
        uint8_t *srow = scales + r * nb;
        for (int b = threadIdx.x; b < nb; b += ROW_THREADS) {
            Block16 x = load_block(row + b * NVFP4_BLOCK);
            if (PROT) {
                const unsigned m = block_mask16(smask, b);
                if (m) clear_protected(x, m);
            }
            u32x2 cw;
            const unsigned sc = quantize_block(x, ts, cw);
            *reinterpret_cast<u32x2 *>(crow + b * 8) = cw;
            srow[b] = (uint8_t)sc;
        }
        if (PROT)
            for (int j = threadIdx.x; j < k; j += ROW_THREADS) side[r * k + j] = row[idx[j]];
    }
}

hipError_t launch_quantize(const uint16_t *A, int64_t R, int64_t K, int64_t lda,
                           const int32_t *idx, int32_t k, const float *alpha, uint8_t *codes,
                           uint8_t *scales, uint16_t *side, hipStream_t s)
{
    if (R == 0 || K == 0) return hipSuccess;
    const unsigned grid = (unsigned)min(R, (int64_t)2048);
    if (k > 0)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid), dim3(ROW_THREADS), 0, s, A, R, K, lda,
                           idx, k, alpha, codes, scales, side);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid), dim3(ROW_THREADS), 0, s, A, R, K,
                           lda, idx, k, alpha, codes, scales, side);
    return hipGetLastError();
}

}  // namespace splice
