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
            // A fragments of this sub-step stay live; B fragments are decoded
            // one at a time and used at once.
            f16x8 af[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; i++)
                af[i] = decode8(xc[i][s], e4m3_pair((xs[i] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const f16x8 bf = decode8(wc[j][s], e4m3_pair((ws[j] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
                for (int i = 0; i < C::FM; i++) acc[i][j] = mfma_f16(af[i], bf, acc[i][j]);
            }
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
            bf16x8 af[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; i++) {
                const int64_t m = m0 + wm * C::WM + i * 16 + rr;
                af[i] = load_bf16x8(a.X_S + m * k + c0, (m < M) ? valid : 0, al);
            }
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const int64_t n = n0 + wn * C::WN + j * 16 + rr;
                const bf16x8 bf = load_bf16x8(a.W_S + n * k + c0, (n < N) ? valid : 0, al);
#pragma unroll
                for (int i = 0; i < C::FM; i++) acc[i][j] = mfma_bf16(af[i], bf, acc[i][j]);
            }
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

// ===========================================================================
// Large-tile prefill path: 256x256 workgroup tile, 4 waves (2x2) of 128x128,
// v_mfma_f32_32x32x16_f16, K step of 64 channels (4 NVFP4 blocks: 32 code
// bytes and 4 scale bytes per row), register-staged double-buffered LDS.
// Lane group g = l/32 owns channels [32g, 32g+32) of a step (one 16-byte code
// chunk, two block scales); MFMA sub-step s takes its channels [32g+8s, +8).
// ===========================================================================
constexpr int BK2 = 64;
constexpr int CODE_ROW2 = BK2 / 2;     // 32 code bytes per row per step
constexpr int SCALE_ROW2 = BK2 / 16;   // 4 scale bytes per row per step

struct Big {
    static constexpr int BM = 256, BN = 256, WM = 128, WN = 128, FM = 4, FN = 4;
    static constexpr int XC = BM * CODE_ROW2, WC = BN * CODE_ROW2;
    static constexpr int XSC = BM * SCALE_ROW2, WSC = BN * SCALE_ROW2;
    static constexpr int STAGE = XC + WC + XSC + WSC;      // 18 KB
};

// 16-byte chunk h (0/1) of row r: 16 consecutive rows land on 16 distinct
// 16-byte slots of the 256-byte bank window
__device__ __forceinline__ int chunk2_off(int r, int h) { return r * CODE_ROW2 + ((h ^ ((r >> 3) & 1)) << 4); }

template <bool TAIL>
__global__ __launch_bounds__(256) void prefill_big_kernel(GemmArgs a)
{
    using C = Big;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, rr = lane & 31;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int tiles_m = (int)((M + C::BM - 1) / C::BM), tiles_n = (int)((N + C::BN - 1) / C::BN);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t rowb = K / 2, rows = K / 16;
    const int nk = (int)(K / BK2);

    // staging: thread t moves code chunks t and t+256 of each operand (row c/2,
    // half c%2) and the 4 scale bytes of row t of each operand
    const int64_t xm0 = m0 + (tid >> 1), xm1 = m0 + ((tid + 256) >> 1);
    const int64_t wn0 = n0 + (tid >> 1), wn1 = n0 + ((tid + 256) >> 1);
    const int hh = tid & 1;
    const uint8_t *px0 = a.Xq + (xm0 < M ? xm0 : 0) * rowb + hh * 16;
    const uint8_t *px1 = a.Xq + (xm1 < M ? xm1 : 0) * rowb + hh * 16;
    const uint8_t *pw0 = a.Wq + (wn0 < N ? wn0 : 0) * rowb + hh * 16;
    const uint8_t *pw1 = a.Wq + (wn1 < N ? wn1 : 0) * rowb + hh * 16;
    const bool okx0 = xm0 < M, okx1 = xm1 < M, okw0 = wn0 < N, okw1 = wn1 < N;
    const int64_t xsr = m0 + tid, wsr = n0 + tid;
    const uint8_t *pxs = a.Xs + (xsr < M ? xsr : 0) * rows;
    const uint8_t *pws = a.Ws + (wsr < N ? wsr : 0) * rows;
    const bool okxs = xsr < M, okws = wsr < N;
    u32x4 sx0, sx1, sw0, sw1;
    unsigned ssx, ssw;
    auto gload = [&](int kt) {
        const int64_t off = (int64_t)kt * CODE_ROW2, soff = (int64_t)kt * SCALE_ROW2;
        sx0 = okx0 ? *reinterpret_cast<const u32x4 *>(px0 + off) : u32x4{0, 0, 0, 0};
        sx1 = okx1 ? *reinterpret_cast<const u32x4 *>(px1 + off) : u32x4{0, 0, 0, 0};
        sw0 = okw0 ? *reinterpret_cast<const u32x4 *>(pw0 + off) : u32x4{0, 0, 0, 0};
        sw1 = okw1 ? *reinterpret_cast<const u32x4 *>(pw1 + off) : u32x4{0, 0, 0, 0};
        ssx = okxs ? *reinterpret_cast<const unsigned *>(pxs + soff) : 0u;
        ssw = okws ? *reinterpret_cast<const unsigned *>(pws + soff) : 0u;
    };
    auto lstore = [&](uint8_t *st) {
        *reinterpret_cast<u32x4 *>(st + chunk2_off(tid >> 1, hh)) = sx0;
        *reinterpret_cast<u32x4 *>(st + chunk2_off((tid + 256) >> 1, hh)) = sx1;
        *reinterpret_cast<u32x4 *>(st + C::XC + chunk2_off(tid >> 1, hh)) = sw0;
        *reinterpret_cast<u32x4 *>(st + C::XC + chunk2_off((tid + 256) >> 1, hh)) = sw1;
        *reinterpret_cast<unsigned *>(st + C::XC + C::WC + tid * SCALE_ROW2) = ssx;
        *reinterpret_cast<unsigned *>(st + C::XC + C::WC + C::XSC + tid * SCALE_ROW2) = ssw;
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[i][j][q] = 0.f;

    // fragment codes/scales of one stage for this wave
    u32x4 xc[C::FM], wc[C::FN];
    unsigned xs[C::FM], ws[C::FN];
    auto lfrag = [&](const uint8_t *st) {
#pragma unroll
        for (int i = 0; i < C::FM; i++) {
            const int r = wm * C::WM + i * 32 + rr;
            xc[i] = *reinterpret_cast<const u32x4 *>(st + chunk2_off(r, g));
            xs[i] = *reinterpret_cast<const uint16_t *>(st + C::XC + C::WC + r * SCALE_ROW2 + 2 * g);
        }
#pragma unroll
        for (int j = 0; j < C::FN; j++) {
            const int r = wn * C::WN + j * 32 + rr;
            wc[j] = *reinterpret_cast<const u32x4 *>(st + C::XC + chunk2_off(r, g));
            ws[j] = *reinterpret_cast<const uint16_t *>(st + C::XC + C::WC + C::XSC + r * SCALE_ROW2 + 2 * g);
        }
    };
    f16x2 xp[C::FM][2], wp[C::FN][2];
    f16x8 af[C::FM], an[C::FM], bf;
    // scale pairs and the first fragments (s = 0, j = 0) of the stage in xc/wc
    auto head = [&]() {
#pragma unroll
        for (int i = 0; i < C::FM; i++) {
            xp[i][0] = e4m3_pair(xs[i] & 0xFFu);
            xp[i][1] = e4m3_pair((xs[i] >> 8) & 0xFFu);
        }
#pragma unroll
        for (int j = 0; j < C::FN; j++) {
            wp[j][0] = e4m3_pair(ws[j] & 0xFFu);
            wp[j][1] = e4m3_pair((ws[j] >> 8) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < C::FM; i++) af[i] = decode8(xc[i][0], xp[i][0]);
        bf = decode8(wc[0][0], wp[0][0]);
    };
    // MFMA step t = 4*s + j of the stage, decoding the operands of step t+1
    auto step = [&](int t) {
        const int s = t >> 2, j = t & 3;
        f16x8 bn = bf;
        if (j + 1 < C::FN) bn = decode8(wc[j + 1][s], wp[j + 1][s >> 1]);
        else if (s + 1 < 4) bn = decode8(wc[0][s + 1], wp[0][(s + 1) >> 1]);
        if (s + 1 < 4) an[j] = decode8(xc[j][s + 1], xp[j][(s + 1) >> 1]);
#pragma unroll
        for (int i = 0; i < C::FM; i++) acc[i][j] = mfma32_f16(af[i], bf, acc[i][j]);
        bf = bn;
        if (j == 3 && s + 1 < 4) {
#pragma unroll
            for (int i = 0; i < C::FM; i++) af[i] = an[i];
        }
    };

    if (nk > 0) {
        gload(0);
        lstore(lds);
        __syncthreads();
        lfrag(lds);
        head();
    }
    for (int kt = 0; kt < nk; kt++) {
        const bool more = kt + 1 < nk;
        if (more) gload(kt + 1);
#pragma unroll
        for (int t = 0; t < 14; t++) step(t);
        // stage kt+1 into the other buffer; its fragments are read while the
        // last MFMAs of this stage drain
        if (more) lstore(lds + ((kt + 1) & 1) * C::STAGE);
        __syncthreads();
        f16x8 a_last[C::FM], b14 = bf;
#pragma unroll
        for (int i = 0; i < C::FM; i++) a_last[i] = af[i];
        const f16x8 b15 = decode8(wc[3][3], wp[3][1]);
        if (more) lfrag(lds + ((kt + 1) & 1) * C::STAGE);
#pragma unroll
        for (int i = 0; i < C::FM; i++) acc[i][2] = mfma32_f16(a_last[i], b14, acc[i][2]);
        if (more) head();
#pragma unroll
        for (int i = 0; i < C::FM; i++) acc[i][3] = mfma32_f16(a_last[i], b15, acc[i][3]);
#pragma unroll
        for (int q = 0; q < 56; q++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
        }
    }

    const float alpha = (*a.alpha_x) * (*a.alpha_w);
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) acc[i][j] *= alpha;
    if (TAIL) {
        const int k = a.k;
        const bool al = (k % 8) == 0;
        for (int kk = 0; kk < k; kk += 16) {
            const int c0 = kk + g * 8;
            const int valid = max(0, min(8, k - c0));
            bf16x8 af[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; i++) {
                const int64_t m = m0 + wm * C::WM + i * 32 + rr;
                af[i] = load_bf16x8(a.X_S + m * k + c0, (m < M) ? valid : 0, al);
            }
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const int64_t n = n0 + wn * C::WN + j * 32 + rr;
                const bf16x8 bf = load_bf16x8(a.W_S + n * k + c0, (n < N) ? valid : 0, al);
#pragma unroll
                for (int i = 0; i < C::FM; i++) acc[i][j] = mfma32_bf16(af[i], bf, acc[i][j]);
            }
        }
    }
    // store: lane writes column (n0 + wn*128 + j*32 + rr) of rows
    // m0 + wm*128 + i*32 + 8*(q/4) + 4*g + q%4
    const int64_t mb = m0 + wm * C::WM + g * 4, nb = n0 + wn * C::WN + rr;
    float *yb = a.Y + mb * a.ldy + nb;
    if (m0 + C::BM <= M && n0 + C::BN <= N) {
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int q = 0; q < 16; q++) {
                float *yr = yb + (int64_t)(i * 32 + (q >> 2) * 8 + (q & 3)) * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++) yr[j * 32] = acc[i][j][q];
            }
    } else {
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int dm = i * 32 + (q >> 2) * 8 + (q & 3);
                if (mb + dm >= M) continue;
                float *yr = yb + (int64_t)dm * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    if (nb + j * 32 < N) yr[j * 32] = acc[i][j][q];
            }
    }
}

// ===========================================================================
// LDS-decode prefill path: each workgroup decodes every NVFP4 element of its
// 256x256 tile exactly once per K step into a swizzled FP16 tile in LDS
// (double buffered, 2 x 64 KB); the four waves (2x2, 128x128 each) read their
// MFMA fragments from it with ds_read_b128 and run v_mfma_f32_32x32x16_f16.
// While a wave multiplies stage kt it decodes its share of stage kt+1 from
// registers (fetched one step earlier) into the other buffer, so decode VALU
// work, global loads and LDS traffic all hide under the matrix cores.
// Decode share per thread and step: 4 units of (row, 32-channel half) = 16
// code bytes + 2 scale bytes -> 32 FP16 values.
// ===========================================================================
struct LdsCfg {
    static constexpr int BM = 256, BN = 256, BKL = 64, WM = 128, WN = 128, FM = 4, FN = 4;
    static constexpr int ROWB = BKL * 2;                 // 128 bytes of FP16 per row
    static constexpr int TILE = (BM + BN) * ROWB;         // 64 KB per stage
};

// byte offset of 16-byte chunk c (8 channels) of row r in an FP16 tile.
// Measured on gfx950: a 16-byte LDS read is served 16 lanes per cycle from a
// 256-byte bank window, a 16-byte write 8 lanes per cycle from a 128-byte
// window.  The chunk swizzle (r%8) ^ ((r/8)%2) puts 16 consecutive rows of a
// fragment read and 8 consecutive rows of a decode write on distinct slots.
__device__ __forceinline__ int f16_off(int r, int c)
{
    return r * LdsCfg::ROWB + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

template <bool TAIL>
__global__ __launch_bounds__(256) void prefill_lds_kernel(GemmArgs a)
{
    using C = LdsCfg;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, rr = lane & 31;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int tiles_m = (int)((M + C::BM - 1) / C::BM), tiles_n = (int)((N + C::BN - 1) / C::BN);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t rowb = K / 2, rows = K / 16;
    const int nk = (int)(K / C::BKL);

    // decode units of this thread: u = tid + 256*i; i = 0,1 -> X rows, 2,3 -> W rows
    const int half = tid & 1;
    int urow[4];
    const uint8_t *ucode[4];
    const uint8_t *uscale[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = ((tid + 256 * (i & 1)) >> 1);            // 0..255 within the operand tile
        const bool isx = i < 2;
        const int64_t gr = (isx ? m0 : n0) + r;
        const int64_t rr0 = gr < (isx ? M : N) ? gr : 0;
        urow[i] = (isx ? 0 : C::BM) + r;                        // row in the combined LDS tile
        ucode[i] = (isx ? a.Xq : a.Wq) + rr0 * rowb + half * 16;
        uscale[i] = (isx ? a.Xs : a.Ws) + rr0 * rows + half * 2;
    }
    u32x4 pc[4];
    unsigned ps[4];
    // Rows past the edge of the operand read its row 0 instead: an A row only
    // reaches output row m and a B row only output column n, and those rows
    // and columns are never stored, so no masking (and no wait) is needed.
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            pc[i] = *reinterpret_cast<const u32x4 *>(ucode[i] + (int64_t)kt * 32);
            ps[i] = *reinterpret_cast<const uint16_t *>(uscale[i] + (int64_t)kt * 4);
        }
    };
    auto decode_store = [&](uint8_t *tile) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f16x2 s0 = e4m3_pair(ps[i] & 0xFFu), s1 = e4m3_pair((ps[i] >> 8) & 0xFFu);
#pragma unroll
            for (int d = 0; d < 4; d++) {
                const f16x8 v = decode8(pc[i][d], d < 2 ? s0 : s1);
                *reinterpret_cast<f16x8 *>(tile + f16_off(urow[i], half * 4 + d)) = v;
            }
        }
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[i][j][q] = 0.f;

    if (nk > 0) {
        gload(0);
        decode_store(lds);
        gload(min(1, nk - 1));
    }
    __syncthreads();
    const int arow = wm * C::WM + rr, brow = C::BM + wn * C::WN + rr;
    auto decode_unit = [&](uint8_t *tile, int i) {
        const f16x2 s0 = e4m3_pair(ps[i] & 0xFFu), s1 = e4m3_pair((ps[i] >> 8) & 0xFFu);
#pragma unroll
        for (int d = 0; d < 4; d++)
            *reinterpret_cast<f16x8 *>(tile + f16_off(urow[i], half * 4 + d)) = decode8(pc[i][d], d < 2 ? s0 : s1);
    };
    for (int kt = 0; kt < nk; kt++) {
        const uint8_t *cur = lds + (kt & 1) * C::TILE;
        uint8_t *nxt = lds + ((kt + 1) & 1) * C::TILE;
        f16x8 a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; i++) a0[i] = *reinterpret_cast<const f16x8 *>(cur + f16_off(arow + i * 32, g));
#pragma unroll
        for (int j = 0; j < C::FN; j++) b0[j] = *reinterpret_cast<const f16x8 *>(cur + f16_off(brow + j * 32, g));
        // Per sub-step: issue the fragment reads of sub-step s+1 first, then the
        // LDS stores of this sub-step's decode unit, then the MFMAs.  LDS
        // operations retire in order, so a wait for those reads never waits
        // for stores queued behind them.
#pragma unroll
        for (int s = 0; s < 4; s++) {
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < C::FM; i++)
                    a1[i] = *reinterpret_cast<const f16x8 *>(cur + f16_off(arow + i * 32, (s + 1) * 2 + g));
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    b1[j] = *reinterpret_cast<const f16x8 *>(cur + f16_off(brow + j * 32, (s + 1) * 2 + g));
            }
            decode_unit(nxt, s);      // on the last step this fills the idle buffer
#pragma unroll
            for (int j = 0; j < C::FN; j++)
#pragma unroll
                for (int i = 0; i < C::FM; i++) acc[i][j] = mfma32_f16(a0[i], b0[j], acc[i][j]);
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < C::FM; i++) a0[i] = a1[i];
#pragma unroll
                for (int j = 0; j < C::FN; j++) b0[j] = b1[j];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        gload(min(kt + 2, nk - 1));
        lds_barrier();      // the prefetch of step kt+2 stays in flight
    }

    const float alpha = (*a.alpha_x) * (*a.alpha_w);
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) acc[i][j] *= alpha;
    if (TAIL) {
        const int k = a.k;
        const bool al = (k % 8) == 0;
        for (int kk = 0; kk < k; kk += 16) {
            const int c0 = kk + g * 8;
            const int valid = max(0, min(8, k - c0));
            bf16x8 af[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; i++) {
                const int64_t m = m0 + wm * C::WM + i * 32 + rr;
                af[i] = load_bf16x8(a.X_S + m * k + c0, (m < M) ? valid : 0, al);
            }
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const int64_t n = n0 + wn * C::WN + j * 32 + rr;
                const bf16x8 bf = load_bf16x8(a.W_S + n * k + c0, (n < N) ? valid : 0, al);
#pragma unroll
                for (int i = 0; i < C::FM; i++) acc[i][j] = mfma32_bf16(af[i], bf, acc[i][j]);
            }
        }
    }
    const int64_t mb = m0 + wm * C::WM + g * 4, nb = n0 + wn * C::WN + rr;
    float *yb = a.Y + mb * a.ldy + nb;
    if (m0 + C::BM <= M && n0 + C::BN <= N) {
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int q = 0; q < 16; q++) {
                float *yr = yb + (int64_t)(i * 32 + (q >> 2) * 8 + (q & 3)) * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++) yr[j * 32] = acc[i][j][q];
            }
    } else {
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int dm = i * 32 + (q >> 2) * 8 + (q & 3);
                if (mb + dm >= M) continue;
                float *yr = yb + (int64_t)dm * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    if (nb + j * 32 < N) yr[j * 32] = acc[i][j][q];
            }
    }
}

template <bool TAIL>
static hipError_t launch_prefill_lds(const GemmArgs &a, hipStream_t s)
{
    const int64_t tiles = ((a.M + LdsCfg::BM - 1) / LdsCfg::BM) * ((a.N + LdsCfg::BN - 1) / LdsCfg::BN);
    const size_t lds = 2 * LdsCfg::TILE;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_lds_kernel<TAIL>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(prefill_lds_kernel<TAIL>, dim3((unsigned)tiles), dim3(256), lds, s, a);
    return hipGetLastError();
}

static hipError_t run_prefill_big(const GemmArgs &a, hipStream_t s)
{
    const int64_t tiles = ((a.M + Big::BM - 1) / Big::BM) * ((a.N + Big::BN - 1) / Big::BN);
    if (a.k > 0)
        hipLaunchKernelGGL(prefill_big_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(prefill_big_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int BM, int BN, bool TAIL>
static hipError_t launch_prefill(const GemmArgs &a, hipStream_t s)
{
    using C = Prefill<BM, BN>;
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const size_t lds = 2 * C::STAGE;
    static bool attr = false;       // raise the dynamic-LDS limit once per instantiation
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_kernel<BM, BN, TAIL>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL((prefill_kernel<BM, BN, TAIL>), dim3((unsigned)tiles), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int BM, int BN>
static hipError_t run_prefill(const GemmArgs &a, hipStream_t s)
{
    return a.k > 0 ? launch_prefill<BM, BN, true>(a, s) : launch_prefill<BM, BN, false>(a, s);
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
        // largest tile that still gives every CU a tile
        const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
        const int64_t t256x128 = ((a.M + 255) / 256) * ((a.N + 127) / 128);
        (void)t256x128;
        if (t256 >= 240) return a.k > 0 ? launch_prefill_lds<true>(a, s) : launch_prefill_lds<false>(a, s);
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
