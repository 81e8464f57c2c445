// gemm.hip -- the two SpliceGEMM datapaths (FourSight, arXiv 2611.04887v1,
// Sec. 4.2 Eq. 5 and Sec. 5.1 "dual-path execution"), built for gfx950.
//
//   Y = (alpha_x * alpha_w) * sum_j deq(Xq)[m,j] deq(Wq)[n,j]  +  X_S W_S^T
//
// Datapath: NVFP4 codes are decoded in registers, exactly, to FP16 (an E2M1
// value times an E4M3 scale has at most 6 significant bits) and multiplied on
// the FP16 matrix cores (v_mfma_f32_16x16x32_f16) into fp32 accumulators.
// The accumulator is then scaled by alpha_x*alpha_w and the BF16 side product
// X_S W_S^T (exact, unscaled protected columns) is accumulated into the same
// registers with v_mfma_f32_16x16x32_bf16 before the single store of Y.
//
// Reduction order inside a K step of 128: lane group g (lanes 16g..16g+15)
// owns channels [32g, 32g+32) of the step, i.e. one 16-byte chunk of codes
// and two block scales per row; MFMA sub-step s consumes its channels
// [32g+8s, 32g+8s+8).  A and B use the same mapping, so this only permutes
// the order of the sum.
#include "common.hpp"
#include "kernels.hpp"

namespace splice {

constexpr int BK = 128;              // channels per K step
constexpr int CODE_ROW = BK / 2;     // 64 code bytes per row per step
constexpr int SCALE_ROW = BK / 16;   // 8 scale bytes per row per step

// ===========================================================================
// Prefill path: 256-thread workgroups (2x2 waves) over BM x BN output tiles,
// codes and scales staged through double-buffered LDS, each wave decoding its
// own fragments from the packed codes.
// ===========================================================================
template <int BM, int BN>
struct Prefill {
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int XC = BM * CODE_ROW, WC = BN * CODE_ROW;
    static constexpr int XSC = BM * SCALE_ROW, WSC = BN * SCALE_ROW;
    static constexpr int STAGE = XC + WC + XSC + WSC;
    static constexpr int XCH = BM * 4 / 256, WCH = BN * 4 / 256;        // 16-B code chunks / thread
    static constexpr int SCR = (BM + BN + 255) / 256;                   // scale rows / thread
};

// position of 16-byte chunk c of row r in LDS (XOR swizzle against bank conflicts)
__device__ __forceinline__ int chunk_off(int r, int c) { return r * CODE_ROW + ((c ^ ((r >> 1) & 3)) << 4); }

// XCD-aware tile order: consecutive workgroups go to different XCDs round
// robin, so each XCD is handed a contiguous range of tiles; inside it tiles
// walk GM tile-rows at a time so neighbours share operand rows in L2.
__device__ __forceinline__ void tile_of(int wg, int nwg, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int q = nwg / 8, r = nwg % 8;
    const int x = wg % 8, local = wg / 8;
    const int tile = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in = tile - group * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

template <int BM, int BN, bool TAIL>
__global__ __launch_bounds__(256) void prefill_kernel(GemmArgs a)
{
    using C = Prefill<BM, BN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t rowb = K / 2, rows = K / 16;
    const int nk = (int)(K / BK);

    // ---- global -> register staging of one K step
    u32x4 xr[C::XCH], wr[C::WCH];
    u32x2 sr[C::SCR];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < C::XCH; i++) {
            const int c = tid + 256 * i, r = c >> 2, cc = c & 3;
            const int64_t m = m0 + r;
            xr[i] = (m < M) ? *reinterpret_cast<const u32x4 *>(a.Xq + m * rowb + (int64_t)kt * CODE_ROW + cc * 16)
                            : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < C::WCH; i++) {
            const int c = tid + 256 * i, r = c >> 2, cc = c & 3;
            const int64_t n = n0 + r;
            wr[i] = (n < N) ? *reinterpret_cast<const u32x4 *>(a.Wq + n * rowb + (int64_t)kt * CODE_ROW + cc * 16)
                            : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < C::SCR; i++) {
            const int r = tid + 256 * i;
            u32x2 v = {0, 0};
            if (r < BM) {
                const int64_t m = m0 + r;
                if (m < M) v = *reinterpret_cast<const u32x2 *>(a.Xs + m * rows + (int64_t)kt * SCALE_ROW);
            } else if (r < BM + BN) {
                const int64_t n = n0 + (r - BM);
                if (n < N) v = *reinterpret_cast<const u32x2 *>(a.Ws + n * rows + (int64_t)kt * SCALE_ROW);
            }
            sr[i] = v;
        }
    };
    auto lstore = [&](uint8_t *st) {
#pragma unroll
        for (int i = 0; i < C::XCH; i++) {
            const int c = tid + 256 * i, r = c >> 2, cc = c & 3;
            *reinterpret_cast<u32x4 *>(st + chunk_off(r, cc)) = xr[i];
        }
#pragma unroll
        for (int i = 0; i < C::WCH; i++) {
            const int c = tid + 256 * i, r = c >> 2, cc = c & 3;
            *reinterpret_cast<u32x4 *>(st + C::XC + chunk_off(r, cc)) = wr[i];
        }
#pragma unroll
        for (int i = 0; i < C::SCR; i++) {
            const int r = tid + 256 * i;
            if (r < BM + BN)
                *reinterpret_cast<u32x2 *>(st + C::XC + C::WC + r * SCALE_ROW) = sr[i];
        }
    };

    f32x4 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
        gload(0);
        lstore(lds);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        uint8_t *cur = lds + (kt & 1) * C::STAGE;
        if (kt + 1 < nk) gload(kt + 1);
        // fragments of this wave
        u32x4 xc[C::FM], wc[C::FN];
        unsigned xs[C::FM], ws[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; i++) {
            const int r = wm * C::WM + i * 16 + rr;
            xc[i] = *reinterpret_cast<const u32x4 *>(cur + chunk_off(r, g));
            xs[i] = *reinterpret_cast<const uint16_t *>(cur + C::XC + C::WC + r * SCALE_ROW + 2 * g);
        }
#pragma unroll
        for (int j = 0; j < C::FN; j++) {
            const int r = wn * C::WN + j * 16 + rr;
            wc[j] = *reinterpret_cast<const u32x4 *>(cur + C::XC + chunk_off(r, g));
            ws[j] = *reinterpret_cast<const uint16_t *>(cur + C::XC + C::WC + C::XSC + r * SCALE_ROW + 2 * g);
        }
#pragma unroll
        for (int s = 0; s < 4; s++) {
            f16x8 af[C::FM], bf[C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; i++)
                af[i] = decode8(xc[i][s], e4m3_pair((xs[i] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
            for (int j = 0; j < C::FN; j++)
                bf[j] = decode8(wc[j][s], e4m3_pair((ws[j] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
            for (int i = 0; i < C::FM; i++)
#pragma unroll
                for (int j = 0; j < C::FN; j++) acc[i][j] = mfma_f16(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) lstore(lds + ((kt + 1) & 1) * C::STAGE);
        __syncthreads();
    }

    // ---- epilogue: scale, BF16 side product, store
    const float alpha = (*a.alpha_x) * (*a.alpha_w);
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) acc[i][j] *= alpha;
    if (TAIL) {
        const int k = a.k;
        const bool al = (k % 8) == 0;
        for (int kk = 0; kk < k; kk += 32) {
            const int c0 = kk + g * 8;
            const int valid = max(0, min(8, k - c0));
            bf16x8 af[C::FM], bf[C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; i++) {
                const int64_t m = m0 + wm * C::WM + i * 16 + rr;
                af[i] = load_bf16x8(a.X_S + m * k + c0, (m < M) ? valid : 0, al);
            }
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const int64_t n = n0 + wn * C::WN + j * 16 + rr;
                bf[j] = load_bf16x8(a.W_S + n * k + c0, (n < N) ? valid : 0, al);
            }
#pragma unroll
            for (int i = 0; i < C::FM; i++)
#pragma unroll
                for (int j = 0; j < C::FN; j++) acc[i][j] = mfma_bf16(af[i], bf[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) {
            const int64_t n = n0 + wn * C::WN + j * 16 + rr;
            if (n >= N) continue;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t m = m0 + wm * C::WM + i * 16 + g * 4 + q;
                if (m < M) a.Y[m * a.ldy + n] = acc[i][j][q];
            }
        }
}

template <int BM, int BN>
static hipError_t run_prefill(const GemmArgs &a, hipStream_t s)
{
    using C = Prefill<BM, BN>;
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const size_t lds = 2 * C::STAGE;
    if (a.k > 0)
        hipLaunchKernelGGL((prefill_kernel<BM, BN, true>), dim3((unsigned)tiles), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL((prefill_kernel<BM, BN, false>), dim3((unsigned)tiles), dim3(256), lds, s, a);
    return hipGetLastError();
}

// ===========================================================================
// Decode path (small M): weight streaming.  A workgroup of four waves owns CB
// column blocks of 16 output channels and a slice of K; its waves split the
// slice, each loading its weight chunks straight from HBM into registers (no
// LDS staging) and the few activation rows from L2, decoding both and
// multiplying on the matrix cores with M padded to MB*16 rows.  The four
// partial accumulators are summed through LDS in wave order.  With one K
// slice the workgroup then scales, adds the BF16 side product and stores Y;
// with several, the unscaled partials go to the workspace and a second kernel
// sums them in slice order.
// ===========================================================================
struct DecodePlan {
    int MB, CB, SK;
};

static DecodePlan decode_plan(int64_t M, int64_t N, int64_t K)
{
    DecodePlan p;
    p.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.CB = p.MB == 1 ? 1 : 2;
    const int64_t nwg = (N + 16 * p.CB - 1) / (16 * p.CB);
    const int64_t chunks = K / BK;
    // split K across workgroups only while the partial sums stay small next to
    // the weight bytes (partials: 8*M*N*SK bytes; weights: 0.5625*N*K)
    int sk = 1;
    while (nwg * sk < 1024 && chunks / (2 * sk) >= 4 && 8.0 * M * (2 * sk) <= 0.1 * 0.5625 * K) sk *= 2;
    p.SK = sk;
    return p;
}

template <int MB, int CB, bool TAIL>
__global__ __launch_bounds__(256) void decode_kernel(GemmArgs a, float *partial)
{
    __shared__ f32x4 red[4][MB * CB][WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t rowb = K / 2, rows = K / 16;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * CB);
    const int SK = gridDim.y;
    const int nchunk = (int)(K / BK);
    const int s0 = (int)((int64_t)blockIdx.y * nchunk / SK), s1 = (int)((int64_t)(blockIdx.y + 1) * nchunk / SK);
    const int cnt = s1 - s0;
    const int c0 = s0 + wave * cnt / 4, c1 = s0 + (wave + 1) * cnt / 4;

    const uint8_t *wrow[CB];
    const uint8_t *wsrow[CB];
    bool wok[CB];
#pragma unroll
    for (int j = 0; j < CB; j++) {
        const int64_t n = n0 + j * 16 + rr;
        wok[j] = n < N;
        wrow[j] = a.Wq + (wok[j] ? n : 0) * rowb + g * 16;
        wsrow[j] = a.Ws + (wok[j] ? n : 0) * rows + 2 * g;
    }
    const uint8_t *xrow[MB];
    const uint8_t *xsrow[MB];
    bool xok[MB];
#pragma unroll
    for (int i = 0; i < MB; i++) {
        const int64_t m = i * 16 + rr;
        xok[i] = m < M;
        xrow[i] = a.Xq + (xok[i] ? m : 0) * rowb + g * 16;
        xsrow[i] = a.Xs + (xok[i] ? m : 0) * rows + 2 * g;
    }

    f32x4 acc[MB][CB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < CB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wc[CB], xc[MB];
    unsigned wsc[CB], xsc[MB];
    auto load = [&](int c, u32x4 *wcv, unsigned *wscv, u32x4 *xcv, unsigned *xscv) {
#pragma unroll
        for (int j = 0; j < CB; j++) {
            wcv[j] = wok[j] ? *reinterpret_cast<const u32x4 *>(wrow[j] + (int64_t)c * CODE_ROW) : u32x4{0, 0, 0, 0};
            wscv[j] = wok[j] ? *reinterpret_cast<const uint16_t *>(wsrow[j] + (int64_t)c * SCALE_ROW) : 0u;
        }
#pragma unroll
        for (int i = 0; i < MB; i++) {
            xcv[i] = xok[i] ? *reinterpret_cast<const u32x4 *>(xrow[i] + (int64_t)c * CODE_ROW) : u32x4{0, 0, 0, 0};
            xscv[i] = xok[i] ? *reinterpret_cast<const uint16_t *>(xsrow[i] + (int64_t)c * SCALE_ROW) : 0u;
        }
    };
    auto compute = [&](const u32x4 *wcv, const unsigned *wscv, const u32x4 *xcv, const unsigned *xscv) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            f16x8 af[MB], bf[CB];
#pragma unroll
            for (int i = 0; i < MB; i++) af[i] = decode8(xcv[i][s], e4m3_pair((xscv[i] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
            for (int j = 0; j < CB; j++) bf[j] = decode8(wcv[j][s], e4m3_pair((wscv[j] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
            for (int i = 0; i < MB; i++)
#pragma unroll
                for (int j = 0; j < CB; j++) acc[i][j] = mfma_f16(af[i], bf[j], acc[i][j]);
        }
    };

    if (c0 < c1) load(c0, wc, wsc, xc, xsc);
    int c = c0;
    for (; c + 1 < c1; c += 2) {
        u32x4 wc2[CB], xc2[MB];
        unsigned wsc2[CB], xsc2[MB];
        load(c + 1, wc2, wsc2, xc2, xsc2);
        compute(wc, wsc, xc, xsc);
        if (c + 2 < c1) load(c + 2, wc, wsc, xc, xsc);
        compute(wc2, wsc2, xc2, xsc2);
    }
    if (c < c1) compute(wc, wsc, xc, xsc);

    // ---- sum the four waves' partials in wave order
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < CB; j++) red[wave][i * CB + j][lane] = acc[i][j];
    __syncthreads();
    const float alpha = (*a.alpha_x) * (*a.alpha_w);
    for (int t = wave; t < MB * CB; t += 4) {
        const int i = t / CB, j = t % CB;
        f32x4 v = red[0][t][lane];
        v += red[1][t][lane];
        v += red[2][t][lane];
        v += red[3][t][lane];
        const int64_t n = n0 + j * 16 + rr;
        if (partial) {
            float *P = partial + (int64_t)blockIdx.y * M * N;
            if (n < N)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int64_t m = i * 16 + g * 4 + q;
                    if (m < M) P[m * N + n] = v[q];
                }
            continue;
        }
        v *= alpha;
        if (TAIL) {
            const int k = a.k;
            const bool al = (k % 8) == 0;
            const int64_t mrow = i * 16 + rr;
            for (int kk = 0; kk < k; kk += 32) {
                const int cc = kk + g * 8;
                const int valid = max(0, min(8, k - cc));
                bf16x8 af = load_bf16x8(a.X_S + mrow * k + cc, (mrow < M) ? valid : 0, al);
                bf16x8 bf = load_bf16x8(a.W_S + n * k + cc, (n < N) ? valid : 0, al);
                v = mfma_bf16(af, bf, v);
            }
        }
        if (n < N)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t m = i * 16 + g * 4 + q;
                if (m < M) a.Y[m * a.ldy + n] = v[q];
            }
    }
}

// Y = alpha * (sum of the K-slice partials in slice order) + X_S W_S^T
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, const float *partial, int SK)
{
    const int64_t M = a.M, N = a.N;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= M * N) return;
    const int64_t m = e / N, n = e - m * N;
    float v = 0.f;
    for (int s = 0; s < SK; s++) v += partial[(int64_t)s * M * N + e];
    v *= (*a.alpha_x) * (*a.alpha_w);
    const int k = a.k;
    for (int i = 0; i < k; i++)
        v = fmaf(__uint_as_float((unsigned)a.X_S[m * k + i] << 16),
                 __uint_as_float((unsigned)a.W_S[n * k + i] << 16), v);
    a.Y[m * a.ldy + n] = v;
}

template <int MB, int CB>
static hipError_t run_decode(const GemmArgs &a, int SK, float *partial, hipStream_t s)
{
    dim3 grid((unsigned)((a.N + 16 * CB - 1) / (16 * CB)), (unsigned)SK);
    if (SK > 1 || a.k == 0)
        hipLaunchKernelGGL((decode_kernel<MB, CB, false>), grid, dim3(256), 0, s, a, SK > 1 ? partial : nullptr);
    else
        hipLaunchKernelGGL((decode_kernel<MB, CB, true>), grid, dim3(256), 0, s, a, (float *)nullptr);
    if (SK > 1) {
        const int64_t total = a.M * a.N;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                           a, partial, SK);
    }
    return hipGetLastError();
}

// ===========================================================================
size_t gemm_ws_bytes(Path p, int64_t M, int64_t N, int64_t K)
{
    if (p != Path::Decode || M == 0 || N == 0) return 0;
    const DecodePlan d = decode_plan(M, N, K);
    return d.SK > 1 ? (size_t)d.SK * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(Path p, const GemmArgs &a, void *ws, size_t, hipStream_t s)
{
    if (a.M == 0 || a.N == 0) return hipSuccess;
    if (p == Path::Prefill) {
        return run_prefill<128, 128>(a, s);
    }
    const DecodePlan d = decode_plan(a.M, a.N, a.K);
    float *partial = static_cast<float *>(ws);
    switch (d.MB) {
    case 1: return run_decode<1, 1>(a, d.SK, partial, s);
    case 2: return run_decode<2, 2>(a, d.SK, partial, s);
    default: return run_decode<4, 2>(a, d.SK, partial, s);
    }
}

}  // namespace splice
