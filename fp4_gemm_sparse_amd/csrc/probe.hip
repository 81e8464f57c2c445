// probe.hip -- measurement aids: the FP16 matrix-core rate this GPU sustains
// (v_mfma_f32_32x32x16_f16, the instruction of the prefill tile), so the
// prefill GEMM can be read against a measured as well as the published peak;
// and the rate of a pure streaming read, the ceiling a weight-streaming decode
// call of the same byte count can reach on this GPU.
#include "common.hpp"
#include "kernels.hpp"

namespace splice {

constexpr int PROBE_WAVES = 4;     // per workgroup; two workgroups per CU -> two waves per SIMD

// Every wave issues `iters` rounds of four independent MFMAs on register
// operands (no memory traffic); lane 0 stores one sum so nothing is removed.
__global__ __launch_bounds__(64 * PROBE_WAVES) void mfma_rate_kernel(int64_t iters, float *sink)
{
    const int lane = threadIdx.x % WAVE;
    const f16x8 a = {(f16)(lane * 0.001f), (f16)0.5f, (f16)0.25f, (f16)0.125f,
                     (f16)1.0f, (f16)-0.5f, (f16)0.75f, (f16)(lane * -0.002f)};
    const f16x8 b = {(f16)0.5f, (f16)(lane * 0.003f), (f16)-0.25f, (f16)0.5f,
                     (f16)0.125f, (f16)1.0f, (f16)(lane * 0.001f), (f16)-1.0f};
    f32x16 acc[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
        for (int q = 0; q < 16; q++) acc[u][q] = 0.f;
    for (int64_t i = 0; i < iters; i++) {
#pragma unroll
        for (int u = 0; u < 4; u++) acc[u] = mfma32_f16(a, b, acc[u]);
    }
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < 4; u++) t += acc[u][0];
    if (lane == 0) sink[blockIdx.x * PROBE_WAVES + threadIdx.x / WAVE] = t;
}

hipError_t launch_mfma_rate(int64_t iters, int64_t workgroups, float *sink, hipStream_t s)
{
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)workgroups), dim3(64 * PROBE_WAVES), 0, s,
                       iters, sink);
    return hipGetLastError();
}

// Pure read: every thread loads READ_UNROLL 16-byte vectors per round, all
// issued before any is used, and folds them into one word; one store per wave
// keeps the loads from being removed.
constexpr int READ_UNROLL = 4;
constexpr int READ_THREADS = 256;

__global__ __launch_bounds__(READ_THREADS) void stream_read_kernel(const u32x4 *src, int64_t n,
                                                                   unsigned *sink)
{
    const int64_t nt = (int64_t)gridDim.x * READ_THREADS;
    unsigned x = 0;
    for (int64_t base = (int64_t)blockIdx.x * READ_THREADS + threadIdx.x; base < n;
         base += nt * READ_UNROLL) {
        u32x4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; u++) {
            const int64_t i = base + u * nt;
            v[u] = i < n ? src[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < READ_UNROLL; u++) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    if (threadIdx.x % WAVE == 0) sink[blockIdx.x * (READ_THREADS / WAVE) + threadIdx.x / WAVE] = x;
}

hipError_t launch_stream_read(const void *src, int64_t bytes, int64_t workgroups, unsigned *sink,
                              hipStream_t s)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(READ_THREADS), 0, s,
                       reinterpret_cast<const u32x4 *>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace splice
