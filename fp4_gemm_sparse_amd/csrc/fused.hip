// fused.hip -- decode SpliceGEMM with the activation preparation in its
// prologue (FourSight, arXiv 2611.04887v1: Sec. 5.1 data preparation and
// dual-path execution; the preparation belongs to the projection's cost as in
// Sec. 6.3, Fig. 10).
//
// For M <= 4 token rows.  A workgroup owns 16*CB output channels and the
// whole K; wave w multiplies K chunks (128 channels) w*CPW .. w*CPW+CPW-1.
//  1. Every independent global load is issued first: the thread's 16-channel
//     blocks of X, its idx entry and its share of the W_S tile ahead of the
//     wave's weight codes and scales.  Loads complete in issue order, so the
//     preparation can start while the weights are still on their way.
//  2. The protected-channel mask is built in LDS from idx.
//  3. Each 16-channel block of the M rows is masked, quantized by one lane
//     with the block functions of nvfp4.hpp that the quantize kernel uses,
//     and decoded into an FP16 copy of X in LDS -- the bits the two-call form
//     would decode from its packed codes.  One lane per block computes the
//     block's scale and keys once; split over two lanes, both would compute
//     them, which measured 5-15% slower on the Qwen3-8B shapes.
//  4. Each wave multiplies its chunks on v_mfma_f32_16x16x32_f16 (A from the
//     LDS copy, B decoded from registers); partial sums meet in LDS in wave
//     order.  The waves that finish a column block add the BF16 side product
//     of X_S (gathered from X through idx) and W_S, both brought in by every
//     thread alike and passed on through LDS: Y = fma(alpha_x*alpha_w, acc,
//     side), as in the two-call kernel.
// With the same wave configuration as the two-call decode kernel for few
// rows (every K <= 4096, and the larger K that kernel takes), the chunk
// split, the MFMA order and the reduction order are the same, and Y is
// bit-identical to it.  Every workgroup repeats the preparation of the
// few rows: that replaces a launch and the HBM round trip of Xq/Xs/X_S.
#include "common.hpp"
#include "kernels.hpp"
#include "nvfp4.hpp"
#include "segments.hpp"

namespace splice {

namespace {

constexpr int FBK = 128;                 // channels per K chunk
constexpr int F_CODE_ROW = FBK / 2;      // code bytes per row per chunk
constexpr int F_SCALE_ROW = FBK / 16;    // scale bytes per row per chunk
constexpr int F_XMAX = 128 * 1024;       // bytes of FP16 activations kept in LDS
constexpr int F_LDS = 160 * 1024;        // LDS of one CU

// eight protected activations row[idx[i]], i < valid (zero beyond), as bf16x8
__device__ __forceinline__ bf16x8 gather_side8(const uint16_t *row, const int32_t *ip, int valid,
                                               int64_t K)
{
    unsigned v[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const int64_t c = e < valid ? ip[e] : -1;
        v[e] = (c >= 0 && c < K) ? row[c] : 0u;
    }
    const u32x4 w = {v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
    return __builtin_bit_cast(bf16x8, w);
}

}  // namespace

template <int NW, int CPW, int CB, int XPT, bool TAIL>
__device__ __forceinline__ void decode_fused_body(const GemmArgs &a, int64_t blk)
{
    // [M][K] FP16 activations, then [NW][CB][64] f32x4 partial sums (the
    // protected-channel mask, and idx when k <= 64, use that space until the
    // main loop), then the W_S and X_S tiles.  XPT: blocks of X per thread
    // loaded up front.
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t rowb = K / 2, rows = K / 16, nb = K / 16;
    const int64_t n0 = blk * (16 * CB);
    const int nchunk = (int)(K / FBK);
    const int k = a.k;
    const int64_t red_off = (M * K * 2 + 15) & ~(int64_t)15;

    // 1. independent global loads: X and idx first, then the weights
    // blocks of X: item q = m * nb + b (fewer than 2^31: M <= 4, K <= 2^14)
    const int items = (int)(M * nb);
    auto blk_ptr = [&](int q) {
        const int m = q / (int)nb;
        return reinterpret_cast<const u32x4 *>(a.X + m * a.ldx + (int64_t)(q - m * (int)nb) * 16);
    };
    u32x4 xv[XPT][2];
#pragma unroll
    for (int j = 0; j < XPT; j++) {
        const int q = tid + j * NT;
        const u32x4 *p = blk_ptr(q < items ? q : 0);
        xv[j][0] = p[0];
        xv[j][1] = p[1];
    }
    const int32_t my_idx = (TAIL && tid < k) ? a.idx[tid] : -1;
    // W_S tile for k = 32 or 64 (CB*16 rows x k): SWD dwords per thread,
    // spread over every thread so that all waves issue the same loads (the
    // compiler can then wait for the weights chunk by chunk); it reaches the
    // waves that finish the column blocks through LDS.  Needed last, but
    // issued before the weights: the preparation below takes long enough to
    // hide its latency, while behind the weights (loads complete in issue
    // order) that latency would land on the kernel's tail -- measured 0.5 us
    // slower on the 4096-channel shapes at one row.
    const bool side_pre = TAIL && (k == 32 || k == 64);
    const int kd = k / 2;                                   // dwords per side row
    constexpr int SWD = (CB * 16 * 32 + NT - 1) / NT;
    unsigned swv[SWD];
    if (side_pre) {
#pragma unroll
        for (int u = 0; u < SWD; u++) {
            const int e = tid + u * NT;
            const int64_t n = n0 + min(e / kd, CB * 16 - 1);
            swv[u] = *reinterpret_cast<const unsigned *>(a.W_S + (n < N ? n : 0) * k + (e % kd) * 2);
        }
    }
    __builtin_amdgcn_sched_barrier(0);     // keep these loads ahead of the weight loads
    const int c0 = wave * CPW;
    u32x4 wc[CPW][CB];
    unsigned ws[CPW][CB];
#pragma unroll
    for (int j = 0; j < CB; j++) {
        const int64_t n = n0 + j * 16 + rr;
        const int64_t nn = n < N ? n : 0;                      // edge rows: never stored
        const uint8_t *pw = a.Wq + nn * rowb + g * 16;
        const uint8_t *ps = a.Ws + nn * rows + 2 * g;
#pragma unroll
        for (int c = 0; c < CPW; c++) {
            const int64_t ci = min(c0 + c, nchunk - 1);        // clamped; skipped at use
            wc[c][j] = *reinterpret_cast<const u32x4 *>(pw + ci * F_CODE_ROW);
            ws[c][j] = *reinterpret_cast<const uint16_t *>(ps + ci * F_SCALE_ROW);
        }
    }
    // 2. protected-channel mask (and, for k <= 64, idx kept in LDS for the
    // side gather, so that gather need not wait for an idx load issued
    // behind the weights)
    uint32_t *smask = reinterpret_cast<uint32_t *>(xl + red_off);
    int32_t *sidx = reinterpret_cast<int32_t *>(xl + red_off + K / 8);     // after the K/32 mask words
    if (TAIL) {
        const int words = (int)((K + 31) / 32);
        for (int i = tid; i < words; i += NT) smask[i] = 0;
        if (side_pre && tid < k) sidx[tid] = my_idx;
        __syncthreads();
        if (my_idx >= 0 && my_idx < K) atomicOr(&smask[my_idx >> 5], 1u << (my_idx & 31));
        for (int i = tid + NT; i < k; i += NT) {
            const int c = a.idx[i];
            if (c >= 0 && c < K) atomicOr(&smask[c >> 5], 1u << (c & 31));
        }
        __syncthreads();
    }

    // 3. quantize and decode the M rows into LDS, one lane per block (block
    // q = m * nb + b lands at byte 32 q of the [M][K] FP16 copy)
    {
        const TensorScale ts = tensor_scale(*a.alpha_x);
        auto prep = [&](const u32x4 v0, const u32x4 v1, int q) {
            Block16 x{{v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w}};
            if (TAIL) {
                const unsigned mk = block_mask16(smask, q % (int)nb);
                if (mk) clear_protected(x, mk);
            }
            u32x2 c;
            const f16x2 sc = e4m3_pair(quantize_block(x, ts, c));
            f16x8 *dst = reinterpret_cast<f16x8 *>(xl + (int64_t)q * 32);
            dst[0] = decode8(c.x, sc);
            dst[1] = decode8(c.y, sc);
        };
#pragma unroll
        for (int j = 0; j < XPT; j++) {
            const int q = tid + j * NT;
            if (q < items) prep(xv[j][0], xv[j][1], q);
        }
        for (int q = tid + XPT * NT; q < items; q += NT) {
            const u32x4 *p = blk_ptr(q);
            prep(p[0], p[1], q);
        }
    }
    // the side tiles' LDS home, after the reduction space: W_S [CB*16][kd]
    // dwords, then X_S [M][k] bf16
    uint32_t *sbuf = reinterpret_cast<uint32_t *>(xl + red_off + NW * CB * WAVE * 16);
    uint16_t *sxb = reinterpret_cast<uint16_t *>(sbuf + CB * 16 * kd);
    unsigned short xsv = 0;
    if (side_pre) {
#pragma unroll
        for (int u = 0; u < SWD; u++)
            if (tid + u * NT < CB * 16 * kd) sbuf[tid + u * NT] = swv[u];
        // one element of X_S per thread, gathered from X through idx: issued
        // behind the weights but by every wave alike, and kept in a register
        // until the main loop is done
        const int e = min(tid, (int)M * k - 1);
        const int64_t c = sidx[e % k];
        xsv = a.X[(e / k) * a.ldx + (c >= 0 && c < K ? c : 0)];
    }
    __syncthreads();

    // 4. the wave's chunks
    f32x4 acc[CB];
#pragma unroll
    for (int j = 0; j < CB; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool xrow = rr < M;
    const uint8_t *xbase = xl + (int64_t)(xrow ? rr : 0) * K * 2 + g * 64;   // lane's 32 channels of a chunk
#pragma unroll
    for (int c = 0; c < CPW; c++) {
        const int ci = c0 + c;
        if (ci < nchunk) {
#pragma unroll
            for (int s = 0; s < 4; s++) {
                f16x8 af = *reinterpret_cast<const f16x8 *>(xbase + (int64_t)ci * FBK * 2 + s * 16);
                if (!xrow) af = f16x8{};
#pragma unroll
                for (int j = 0; j < CB; j++) {
                    const f16x8 bf = decode8(wc[c][j][s], e4m3_pair((ws[c][j] >> ((s >> 1) * 8)) & 0xFFu));
                    acc[j] = mfma_f16(af, bf, acc[j]);
                }
            }
        }
    }

    // 5. wave-order reduction, scale, side product, store
    f32x4 *red = reinterpret_cast<f32x4 *>(xl + red_off);
#pragma unroll
    for (int j = 0; j < CB; j++) red[(wave * CB + j) * WAVE + lane] = acc[j];
    if (side_pre && tid < M * k) sxb[tid] = xsv;
    __syncthreads();
    if (wave < CB) {
        const int j = wave;
        f32x4 v = red[j * WAVE + lane];
#pragma unroll
        for (int w = 1; w < NW; w++) v += red[(w * CB + j) * WAVE + lane];
        const float alpha = (*a.alpha_x) * (*a.alpha_w);
        const int64_t n = n0 + j * 16 + rr;
        if (side_pre) {
            // the side product from zero, then Y = fma(alpha, acc, side): the
            // two-call kernel's arithmetic.  Lane (g, rr): row rr, channels
            // 32h + 8g .. +8
            const bf16x8 z = {};
            const bool okm = rr < M, okn = n < N;
            const uint32_t *wrow = sbuf + (j * 16 + rr) * kd;
            const uint16_t *xrow = sxb + (okm ? rr : 0) * k;
            f32x4 side = {0.f, 0.f, 0.f, 0.f};
            for (int h = 0; h < k / 32; h++) {
                const bf16x8 ta = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xrow + 32 * h + 8 * g));
                const bf16x8 tb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wrow + 16 * h + 4 * g));
                side = mfma_bf16(okm ? ta : z, okn ? tb : z, side);
            }
#pragma unroll
            for (int q = 0; q < 4; q++) v[q] = __builtin_fmaf(alpha, v[q], side[q]);
        } else {
            v *= alpha;
        }
        if (TAIL && !side_pre) {          // other k: gathered and direct loads, masked
            const bool al = (k % 8) == 0;
            const int64_t mrow = rr;
            const uint16_t *xr = a.X + (mrow < M ? mrow : 0) * a.ldx;
            for (int kk = 0; kk < k; kk += 32) {
                const int cc = kk + g * 8;
                const int valid = max(0, min(8, k - cc));
                const bf16x8 af = gather_side8(xr, a.idx + cc, (mrow < M) ? valid : 0, K);
                const bf16x8 bf = load_bf16x8(a.W_S + n * k + cc, (n < N) ? valid : 0, al);
                v = mfma_bf16(af, bf, v);
            }
        }
        if (n < N)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t m = g * 4 + q;
                if (m < M) a.Y[m * a.ldy + n] = v[q];
            }
    }
}

template <int NW, int CPW, int CB, int XPT, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode_fused_kernel(GemmArgs a)
{
    decode_fused_body<NW, CPW, CB, XPT, TAIL>(a, blockIdx.x);
}

// over column segments (the projections that read the same rows of X)
template <int NW, int CPW, int CB, int XPT, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode_fused_seg_kernel(SegTable t)
{
    int local;
    const GemmArgs a = seg_args(t, blockIdx.x, local);
    decode_fused_body<NW, CPW, CB, XPT, TAIL>(a, local);
}

template <int NW, int CPW, int CB, int XPT, bool TAIL>
static hipError_t launch_fused(const GemmArgs &a, const SegSpec *sp, size_t lds, int lds_max, hipStream_t s)
{
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_fused_kernel<NW, CPW, CB, XPT, TAIL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds_max);
    static const hipError_t attr_seg = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_fused_seg_kernel<NW, CPW, CB, XPT, TAIL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds_max);
    if (attr != hipSuccess) return attr;
    if (attr_seg != hipSuccess) return attr_seg;
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, 16 * CB);
        hipLaunchKernelGGL((decode_fused_seg_kernel<NW, CPW, CB, XPT, TAIL>), dim3((unsigned)t.start[t.nseg]),
                           dim3(64 * NW), lds, s, t);
    } else {
        hipLaunchKernelGGL((decode_fused_kernel<NW, CPW, CB, XPT, TAIL>),
                           dim3((unsigned)((a.N + 16 * CB - 1) / (16 * CB))), dim3(64 * NW), lds, s, a);
    }
    return hipGetLastError();
}

template <int NW, int CPW, int CB, int XPT>
static hipError_t run_fused_x(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    constexpr int red_bytes = NW * CB * WAVE * 16;
    constexpr int side_bytes = (CB * 16 + 4) * 128;                  // W_S and X_S tiles, k <= 64
    constexpr int lds_max = 4 * (NW * CPW * FBK) * 2 + red_bytes + side_bytes;   // largest M and K
    static_assert(lds_max <= F_LDS, "fused decode LDS budget");
    const size_t lds = (size_t)((a.M * a.K * 2 + 15) & ~(int64_t)15) + red_bytes + (a.k > 0 ? side_bytes : 0);
    if (a.k > 0) return launch_fused<NW, CPW, CB, XPT, true>(a, sp, lds, lds_max, s);
    return launch_fused<NW, CPW, CB, XPT, false>(a, sp, lds, lds_max, s);
}

// 16-channel blocks of X per thread loaded ahead of the weights: all of them
// when they are at most four, else the first four
template <int NW, int CPW, int CB>
static hipError_t run_fused(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    const int64_t items = a.M * a.K / 16;
    if (items <= 64 * NW) return run_fused_x<NW, CPW, CB, 1>(a, sp, s);
    if (items <= 2 * 64 * NW) return run_fused_x<NW, CPW, CB, 2>(a, sp, s);
    return run_fused_x<NW, CPW, CB, 4>(a, sp, s);
}

// The FP16 copy of the M rows must fit the LDS budget and K must be whole
// 128-channel chunks, at most 16 waves x 8 chunks.
bool fused_decode_ok(int64_t M, int64_t K)
{
    return M >= 1 && M <= 4 && K >= FBK && K % FBK == 0 && K <= 16 * 8 * FBK && M * K * 2 <= F_XMAX;
}

// Wave configurations from sweeps on MI355X (Qwen3-8B shapes, graph replay,
// weights streamed from HBM).  K <= 4096: the two-call kernel's eight waves of
// four chunks (the two forms then agree bit for bit), with 48 columns per
// workgroup for wide N at two or more rows, so that fewer workgroups repeat
// the preparation (at two and four rows 8-18% faster than sixteen waves of
// two chunks, once each lane quantizes whole blocks).  Larger K: the two-call
// kernel's configurations.  The column grouping leaves each column's
// arithmetic as it is, so a call over several weight matrices gives the bits
// of one call per matrix.
// configuration choice for a.N columns (the sum of the widths when sp is set)
static hipError_t dispatch_fused(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    const int nchunk = (int)(a.K / FBK);
    const int64_t colblocks = (a.N + 15) / 16;
    if (nchunk <= 8 * 4)
        return (a.M > 1 && colblocks >= 512) ? run_fused<8, 4, 3>(a, sp, s) : run_fused<8, 4, 1>(a, sp, s);
    if (nchunk <= 16 * 4) return run_fused<16, 4, 1>(a, sp, s);
    if (nchunk <= 16 * 6) return run_fused<16, 6, 1>(a, sp, s);
    return run_fused<16, 8, 1>(a, sp, s);
}

hipError_t launch_gemm_fused(const GemmArgs &a, hipStream_t s)
{
    if (a.M == 0 || a.N == 0) return hipSuccess;
    if (a.K == 0) return launch_gemm(Path::Prefill, a, nullptr, 0, s);   // Y = 0 (k <= K)
    return dispatch_fused(a, nullptr, s);
}

hipError_t launch_gemm_fused_seg(const GemmArgs &a, const GemmSeg *seg, int nseg, hipStream_t s)
{
    GemmArgs b = a;
    b.N = 0;
    for (int i = 0; i < nseg; i++) b.N += seg[i].N;
    if (nseg == 0 || b.M == 0 || b.N == 0) return hipSuccess;
    if (b.K == 0) return launch_gemm_seg(Path::Prefill, b, seg, nseg, nullptr, s);   // Y = 0 (k <= K)
    const SegSpec sp{seg, nseg};
    return dispatch_fused(b, &sp, s);
}

}  // namespace splice
