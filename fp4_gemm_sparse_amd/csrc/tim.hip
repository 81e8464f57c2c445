// tim.hip -- TIM-aware sequence filtering (FourSight, arXiv 2611.04887v1,
// Sec. 4.1 "dual-gate mechanism", Eq. 3-4; settings in Sec. 6.1).
//
// A token of sequence i is a tail token when its training-policy
// log-probability is <= log(tau).  G1 = number of tail tokens, G2 = longest
// run of consecutive tail tokens; the sequence is kept when
// G1 * k1_den < k1_num * len (K1 = k1_num/k1_den x len) and G2 < K2, and its
// advantages are multiplied by that indicator in place.
//
// One workgroup per sequence, NW waves over contiguous 256-token segments
// (16 for rows longer than 1024 tokens, so that an 8k response takes at most
// two steps per wave), four tokens per lane (one 16-byte load when the row
// allows it).
// A stretch of tokens is summarised by (count, leading tail run, trailing
// tail run, longest run, length); that summary combines associatively in
// order, so a butterfly over the lanes (left operand from the lower lanes)
// gives each 256-token chunk's summary, a running fold gives the segment's,
// and thread 0 folds the segments in wave order.  Integer results only:
// identical to a sequential scan.
#include "common.hpp"
#include "kernels.hpp"

namespace splice {

namespace {

constexpr int TIM_CHUNK = 256;     // tokens per wave step (4 per lane)

struct RunSum {
    int cnt, lead, trail, best, len;
};

__device__ __forceinline__ RunSum run_combine(const RunSum &a, const RunSum &b)
{
    RunSum r;
    r.cnt = a.cnt + b.cnt;
    r.lead = (a.lead == a.len) ? a.len + b.lead : a.lead;
    r.trail = (b.trail == b.len) ? b.len + a.trail : b.trail;
    r.best = max(max(a.best, b.best), a.trail + b.lead);
    r.len = a.len + b.len;
    return r;
}

// summary of four tokens, tail flags in bits 0..3 (bit 0 first)
__device__ __forceinline__ RunSum run_of4(unsigned b)
{
    RunSum r;
    r.cnt = __popc(b);
    r.lead = __builtin_ctz(~b);                        // <= 4: bit 4 of ~b is set
    r.trail = __builtin_clz(~(b << 28));               // ones down from bit 3
    unsigned m = b;
    int n = 0;
    while (m) {
        m &= m >> 1;
        n++;
    }
    r.best = n;
    r.len = 4;
    return r;
}

__device__ __forceinline__ RunSum shfl_xor(const RunSum &v, int d)
{
    return RunSum{__shfl_xor(v.cnt, d), __shfl_xor(v.lead, d), __shfl_xor(v.trail, d),
                  __shfl_xor(v.best, d), __shfl_xor(v.len, d)};
}

// the summary of one 256-token chunk, in every lane of the wave
__device__ __forceinline__ RunSum chunk_summary(unsigned b)
{
    const int lane = threadIdx.x % WAVE;
    RunSum s = run_of4(b);
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const RunSum o = shfl_xor(s, d);
        s = (lane & d) ? run_combine(o, s) : run_combine(s, o);
    }
    return s;
}

}  // namespace

template <int NW, bool VEC>
__global__ __launch_bounds__(64 * NW) void tim_filter_kernel(TimArgs a)
{
    __shared__ RunSum part[NW];
    const int64_t i = blockIdx.x;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int64_t n = min(max((int64_t)a.len[i], (int64_t)0), a.ldl);
    const float *row = a.logp + i * a.ldl;
    const float thr = a.log_tau;
    const int64_t chunks = (n + TIM_CHUNK - 1) / TIM_CHUNK;
    const int64_t per = (chunks + NW - 1) / NW;
    const int64_t c0 = min(chunks, (int64_t)wave * per), c1 = min(chunks, c0 + per);

    auto tail_bits = [&](int64_t c) -> unsigned {
        const int64_t t = c * TIM_CHUNK + lane * 4;
        unsigned b = 0;
        if (VEC && t + 4 <= n) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(row + t);
            b = (v[0] <= thr ? 1u : 0u) | (v[1] <= thr ? 2u : 0u) | (v[2] <= thr ? 4u : 0u) |
                (v[3] <= thr ? 8u : 0u);
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (t + j < n && row[t + j] <= thr) b |= 1u << j;
        }
        return b;
    };

    RunSum run{0, 0, 0, 0, 0};
    constexpr int U = 4;                       // chunks whose loads are in flight together
    for (int64_t c = c0; c < c1; c += U) {
        unsigned b[U];
#pragma unroll
        for (int u = 0; u < U; u++) b[u] = (c + u < c1) ? tail_bits(c + u) : 0u;
#pragma unroll
        for (int u = 0; u < U; u++)
            if (c + u < c1) run = run_combine(run, chunk_summary(b[u]));
    }
    if (lane == 0) part[wave] = run;
    __syncthreads();
    __shared__ int s_keep;
    if (threadIdx.x == 0) {
        RunSum tot = part[0];
        for (int w = 1; w < NW; w++) tot = run_combine(tot, part[w]);
        const bool keep = ((int64_t)tot.cnt * a.k1_den < a.k1_num * n) && ((int64_t)tot.best < a.k2);
        if (a.keep) a.keep[i] = (uint8_t)keep;
        if (a.g1) a.g1[i] = tot.cnt;
        if (a.g2) a.g2[i] = tot.best;
        s_keep = keep;
    }
    __syncthreads();
    if (!s_keep && a.adv)
        for (int64_t c = threadIdx.x; c < a.adv_cols; c += 64 * NW) a.adv[i * a.lda + c] = 0.0f;
}

template <int NW>
static hipError_t run_tim(const TimArgs &a, hipStream_t s)
{
    const bool vec = (reinterpret_cast<uintptr_t>(a.logp) % 16 == 0) && (a.ldl % 4 == 0);
    if (vec)
        hipLaunchKernelGGL((tim_filter_kernel<NW, true>), dim3((unsigned)a.B), dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((tim_filter_kernel<NW, false>), dim3((unsigned)a.B), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tim_filter(const TimArgs &a, hipStream_t s)
{
    if (a.B == 0) return hipSuccess;
    return a.ldl > 4 * TIM_CHUNK ? run_tim<16>(a, s) : run_tim<4>(a, s);
}

}  // namespace splice
