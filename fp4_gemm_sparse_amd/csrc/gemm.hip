// gemm.hip -- the two SpliceGEMM datapaths (FourSight, arXiv 2611.04887v1,
// Sec. 4.2 Eq. 5 and Sec. 5.1 "dual-path execution"), built for gfx950.
//
//   Y = (alpha_x * alpha_w) * sum_j deq(Xq)[m,j] deq(Wq)[n,j]  +  X_S W_S^T
//
// Datapath: NVFP4 codes are decoded exactly to FP16 (an E2M1 value times an
// E4M3 scale has at most 6 significant bits) and multiplied on the FP16 matrix
// cores (v_mfma_f32_32x32x16_f16 in the 256x256 prefill tile,
// v_mfma_f32_16x16x32_f16 elsewhere) into fp32 accumulators.  The BF16 side
// product X_S W_S^T of the exact, unscaled protected columns runs on the BF16
// matrix cores and is added to alpha_x*alpha_w times the FP4 accumulator
// before the single store of Y.
//
// Reduction order: each MFMA consumes whole 8-channel pieces of one or two
// NVFP4 blocks, A and B with the same channel mapping, so the hardware order
// only permutes the terms of each dot product; K steps are summed in order.
#include "common.hpp"
#include "kernels.hpp"
#include "segments.hpp"

namespace splice {

constexpr int BK = 128;              // channels per decode-path K chunk
constexpr int CODE_ROW = BK / 2;     // 64 code bytes per row per chunk
constexpr int SCALE_ROW = BK / 16;   // 8 scale bytes per row per chunk

// ===========================================================================
// Prefill path
// ===========================================================================
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

// ===========================================================================
// LDS-decode prefill tile: each workgroup decodes every NVFP4 element of its
// tile exactly once per K step (64 channels) into a swizzled FP16 tile in LDS
// (double buffered).  The main form is 256 x 256 with eight waves (2 x 4,
// 128 x 64 each, two per SIMD, 2 x 64 KB of LDS); grids too small for it use
// 128 x 128 with four waves of 64 x 64 (two workgroups per CU).  Waves read
// their MFMA fragments with ds_read_b128 and run v_mfma_f32_32x32x16_f16.
// While a wave multiplies stage kt it decodes its share of stage kt+1 from
// registers (fetched one step earlier) into the other buffer; the second wave
// on each SIMD keeps the matrix core busy while the first decodes, waits for
// LDS or sits at a barrier.
// Decode share per thread and step (both forms): 2 units of (row, 32-channel
// half) = 32 code bytes + 4 scale bytes -> 64 FP16 values.
// ===========================================================================
struct LdsCfg {
    static constexpr int BKL = 64;
    static constexpr int ROWB = BKL * 2;                 // 128 bytes of FP16 per row
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

// Each thread decodes one 8-channel piece of each of its two units per
// sub-step.
// Geometry of an LDS-decode tile: BM x BN outputs, WGM x WGN waves of
// (BM/WGM) x (BN/WGN), K step BKL channels, BM + BN FP16 rows per stage.
template <int BM_, int BN_, int WGM, int WGN>
struct LdsGeo {
    static constexpr int BM = BM_, BN = BN_, BKL = LdsCfg::BKL;
    static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    static constexpr int NT = 64 * WGM * WGN;                  // threads
    static constexpr int ROWS = BM + BN;
    static constexpr int UNITS = ROWS * 2 / NT;                // decode units per thread
    static constexpr int TILE = ROWS * LdsCfg::ROWB;           // bytes per stage
    static_assert(UNITS * NT == ROWS * 2 && FM * 32 == WM && FN * 32 == WN, "tile geometry");
};
// One BM x BN output tile (tm, tn) with WGM x WGN waves (see LdsGeo).
template <int BM, int BN, int WGM, int WGN, bool TAIL>
__device__ __forceinline__ void lds_tile(const GemmArgs &a, int tm, int tn, uint8_t *lds)
{
    using C = LdsGeo<BM, BN, WGM, WGN>;
    constexpr int NT = C::NT, UNITS = C::UNITS;
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 5, rr = lane & 31;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t rowb = K / 2, rows = K / 16;
    const int nk = (int)(K / C::BKL);

    // decode units of this thread: unit i = LDS row (tid + NT*i)/2 (X rows
    // first, then W rows), channel half tid%2.  Rows past the edge read row 0
    // (never stored).
    const int half = tid & 1;
    int urow[UNITS];
    const uint8_t *ucode[UNITS];
    const uint8_t *uscale[UNITS];
#pragma unroll
    for (int i = 0; i < UNITS; i++) {
        const int row = (tid + NT * i) >> 1;
        const bool isx = row < C::BM;
        const int r = isx ? row : row - C::BM;
        const int64_t gr = (isx ? m0 : n0) + r;
        const int64_t rr0 = gr < (isx ? M : N) ? gr : 0;
        urow[i] = row;
        ucode[i] = (isx ? a.Xq : a.Wq) + rr0 * rowb + half * 16;
        uscale[i] = (isx ? a.Xs : a.Ws) + rr0 * rows + half * 2;
    }
    u32x4 pc[UNITS];
    unsigned ps[UNITS];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < UNITS; i++) {
            pc[i] = *reinterpret_cast<const u32x4 *>(ucode[i] + (int64_t)kt * 32);
            ps[i] = *reinterpret_cast<const uint16_t *>(uscale[i] + (int64_t)kt * 4);
        }
    };
    // piece d (8 channels) of every unit into `tile`
    auto decode_piece = [&](uint8_t *tile, int d) {
#pragma unroll
        for (int i = 0; i < UNITS; i++) {
            const f16x2 sc = e4m3_pair(d < 2 ? (ps[i] & 0xFFu) : ((ps[i] >> 8) & 0xFFu));
            *reinterpret_cast<f16x8 *>(tile + f16_off(urow[i], half * 4 + d)) = decode8(pc[i][d], sc);
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
#pragma unroll
        for (int d = 0; d < 4; d++) decode_piece(lds, d);
        gload(min(1, nk - 1));
    }
    __syncthreads();
    const int arow = wm * C::WM + rr, brow = C::BM + wn * C::WN + rr;
    for (int kt = 0; kt < nk; kt++) {
        const uint8_t *cur = lds + (kt & 1) * C::TILE;
        uint8_t *nxt = lds + ((kt + 1) & 1) * C::TILE;
        f16x8 a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; i++) a0[i] = *reinterpret_cast<const f16x8 *>(cur + f16_off(arow + i * 32, g));
#pragma unroll
        for (int j = 0; j < C::FN; j++) b0[j] = *reinterpret_cast<const f16x8 *>(cur + f16_off(brow + j * 32, g));
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
            decode_piece(nxt, s);     // on the last step this fills the idle buffer
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

    // ---- epilogue: Y = alpha_x*alpha_w * acc + X_S W_S^T
    // The side operands (k a multiple of 16) go through the idle LDS stage
    // buffers in passes of up to 128 channels, 64 per buffer, in the same
    // swizzled 128-byte-row layout; all loads of a buffer are issued before its
    // stores (rows past M or N clamped, channels past k re-reading the last
    // ones: neither reaches a stored output).  Per 32-row fragment the side
    // product goes into a small separate accumulator and the first pass stores
    // Y = fma(alpha, acc, side), so the FP4 accumulator is only read; further
    // passes (k > 128) add their side products into Y.
    const float alpha = (*a.alpha_x) * (*a.alpha_w);
    const int k = TAIL ? a.k : 0;
    const int64_t mb = m0 + wm * C::WM + g * 4, nb = n0 + wn * C::WN + rr;
    float *yb = a.Y + mb * a.ldy + nb;
    const bool full = m0 + C::BM <= M && n0 + C::BN <= N;
    auto store_rows = [&](int i, const f32x16 (&v)[C::FN], bool add) {
        if (full) {
#pragma unroll
            for (int q = 0; q < 16; q++) {
                float *yr = yb + (int64_t)(i * 32 + (q >> 2) * 8 + (q & 3)) * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++) yr[j * 32] = add ? yr[j * 32] + v[j][q] : v[j][q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int dm = i * 32 + (q >> 2) * 8 + (q & 3);
                if (mb + dm >= M) continue;
                float *yr = yb + (int64_t)dm * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    if (nb + j * 32 < N) yr[j * 32] = add ? yr[j * 32] + v[j][q] : v[j][q];
            }
        }
    };
    const bool staged = TAIL && k > 0 && k % 16 == 0;
    auto stage = [&](int kp, int kn) {
        constexpr int RS = NT / 8, PU = C::ROWS * 8 / NT;   // rows r0 + RS*u, chunk cc
        const int r0 = tid >> 3, cc = tid & 7;
        const uint16_t *xp = a.X_S + cc * 8, *wp = a.W_S + cc * 8;
        for (int ch = 0; ch * C::BKL < kn; ch++) {
            const int c = min(kp + ch * C::BKL + cc * 8, k - 8) - cc * 8;
            u32x4 v[PU];
#pragma unroll
            for (int u = 0; u < PU; u++) {
                const int row = r0 + RS * u;
                v[u] = row < C::BM ? *reinterpret_cast<const u32x4 *>(xp + min(m0 + row, M - 1) * k + c)
                                   : *reinterpret_cast<const u32x4 *>(wp + min(n0 + row - C::BM, N - 1) * k + c);
            }
#pragma unroll
            for (int u = 0; u < PU; u++)
                *reinterpret_cast<u32x4 *>(lds + ch * C::TILE + f16_off(r0 + RS * u, cc)) = v[u];
        }
        lds_barrier();
    };
    auto side_staged = [&](int i, int kn, f32x16 (&side)[C::FN]) {
        for (int s = 0; s < kn / 16; s++) {
            const uint8_t *tile = lds + (s >> 2) * C::TILE;
            const int c = 2 * (s & 3) + g;
            const bf16x8 af = *reinterpret_cast<const bf16x8 *>(tile + f16_off(arow + i * 32, c));
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const bf16x8 bf = *reinterpret_cast<const bf16x8 *>(tile + f16_off(brow + j * 32, c));
                side[j] = mfma32_bf16(af, bf, side[j]);
            }
        }
    };
    const int kn0 = staged ? min(2 * C::BKL, k) : 0;
    if (staged) stage(0, kn0);
#pragma unroll
    for (int i = 0; i < C::FM; i++) {
        f32x16 side[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) side[j][q] = 0.f;
        if (staged) {
            side_staged(i, kn0, side);
        } else if (TAIL && k > 0) {     // k not a multiple of 16: direct loads, masked
            const bool al = (k % 8) == 0;
            const int64_t m = m0 + wm * C::WM + i * 32 + rr;
            for (int kk = 0; kk < k; kk += 16) {
                const int c0 = kk + g * 8;
                const int valid = max(0, min(8, k - c0));
                const bf16x8 af = load_bf16x8(a.X_S + m * k + c0, (m < M) ? valid : 0, al);
#pragma unroll
                for (int j = 0; j < C::FN; j++) {
                    const int64_t n = n0 + wn * C::WN + j * 32 + rr;
                    const bf16x8 bf = load_bf16x8(a.W_S + n * k + c0, (n < N) ? valid : 0, al);
                    side[j] = mfma32_bf16(af, bf, side[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < C::FN; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) side[j][q] = __builtin_fmaf(alpha, acc[i][j][q], side[j][q]);
        store_rows(i, side, false);
    }
    if (staged)
        for (int kp = 2 * C::BKL; kp < k; kp += 2 * C::BKL) {
            const int kn = min(2 * C::BKL, k - kp);
            lds_barrier();                                  // previous pass fully read
            stage(kp, kn);
            for (int i = 0; i < C::FM; i++) {
                f32x16 side[C::FN];
#pragma unroll
                for (int j = 0; j < C::FN; j++)
#pragma unroll
                    for (int q = 0; q < 16; q++) side[j][q] = 0.f;
                side_staged(i, kn, side);
                store_rows(i, side, true);
            }
        }
}

template <bool TAIL>
__global__ __launch_bounds__(512) void prefill_lds_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((a.M + 255) / 256), tiles_n = (int)((a.N + 255) / 256);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    lds_tile<256, 256, 2, 4, TAIL>(a, tm, tn, lds);
}

// 128 x 128 tiles, four waves of 64 x 64 (two workgroups per CU): for grids
// too small for the 256 x 256 tile
template <bool TAIL>
__global__ __launch_bounds__(256) void prefill_lds128_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((a.M + 127) / 128), tiles_n = (int)((a.N + 127) / 128);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    lds_tile<128, 128, 2, 2, TAIL>(a, tm, tn, lds);
}

// the same tiles over column segments: tile columns numbered across them
template <int BT, int WGN, bool TAIL>
__global__ __launch_bounds__(64 * 2 * WGN) void prefill_seg_kernel(SegTable t)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((t.a.M + BT - 1) / BT);
    int tm, tn, local;
    tile_of(blockIdx.x, gridDim.x, tiles_m, t.start[t.nseg], tm, tn);
    const GemmArgs a = seg_args(t, tn, local);
    lds_tile<BT, BT, 2, WGN, TAIL>(a, tm, local, lds);
}

// ---------------------------------------------------------------------------
// Grouped form (independent products sharing N, K and k, e.g. the experts of
// a MoE layer): one launch covers the tiles of up to GROUP_MAX groups.  The
// group descriptors travel by value in the kernel arguments, so the launch
// needs no device-side table (and can be captured in a graph); workgroup w
// belongs to the group whose tile range [tile_start[e], tile_start[e+1])
// holds w.
// ---------------------------------------------------------------------------
constexpr int GROUP_MAX = 32;

struct GroupDesc {
    const uint8_t *Xq, *Xs;
    const float *alpha_x;
    const uint16_t *X_S;
    const uint8_t *Wq, *Ws;
    const float *alpha_w;
    const uint16_t *W_S;
    float *Y;
    int64_t M;
};

struct GroupedArgs {
    GroupDesc g[GROUP_MAX];
    int tile_start[GROUP_MAX + 1];
    int64_t N, K;
    int k, tiles_n, G;
};

template <int BM, int BN, bool TAIL>
__global__ __launch_bounds__(256) void grouped_prefill_kernel(GroupedArgs ga)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int w = blockIdx.x;
    int e = 0;
    while (e + 1 < ga.G && w >= ga.tile_start[e + 1]) e++;
    const int local = w - ga.tile_start[e];
    const GroupDesc &d = ga.g[e];
    const GemmArgs a{d.Xq, d.Xs, d.alpha_x, d.X_S, d.Wq, d.Ws, d.alpha_w, d.W_S,
                     d.M, ga.N, ga.K, ga.k, d.Y, ga.N};
    lds_tile<BM, BN, 2, 2, TAIL>(a, local / ga.tiles_n, local % ga.tiles_n, lds);
}

template <bool TAIL>
static hipError_t launch_prefill_lds(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    using C = LdsGeo<256, 256, 2, 4>;
    const size_t lds = 2 * C::TILE;
    // raise the dynamic-LDS limit once per instantiation (thread-safe static init)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&prefill_lds_kernel<TAIL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    static const hipError_t attr_seg = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&prefill_seg_kernel<256, 4, TAIL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    if (attr_seg != hipSuccess) return attr_seg;
    const int64_t tiles_m = (a.M + C::BM - 1) / C::BM;
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, C::BN);
        hipLaunchKernelGGL((prefill_seg_kernel<256, 4, TAIL>), dim3((unsigned)(tiles_m * t.start[t.nseg])),
                           dim3(C::NT), lds, s, t);
    } else {
        const int64_t tiles = tiles_m * ((a.N + C::BN - 1) / C::BN);
        hipLaunchKernelGGL(prefill_lds_kernel<TAIL>, dim3((unsigned)tiles), dim3(C::NT), lds, s, a);
    }
    return hipGetLastError();
}

template <bool TAIL>
static hipError_t launch_prefill_lds128(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    using C = LdsGeo<128, 128, 2, 2>;
    const size_t lds = 2 * C::TILE;
    const int64_t tiles_m = (a.M + C::BM - 1) / C::BM;
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, C::BN);
        hipLaunchKernelGGL((prefill_seg_kernel<128, 2, TAIL>), dim3((unsigned)(tiles_m * t.start[t.nseg])),
                           dim3(C::NT), lds, s, t);
    } else {
        const int64_t tiles = tiles_m * ((a.N + C::BN - 1) / C::BN);
        hipLaunchKernelGGL(prefill_lds128_kernel<TAIL>, dim3((unsigned)tiles), dim3(C::NT), lds, s, a);
    }
    return hipGetLastError();
}


template <bool TAIL>
static hipError_t launch_grouped_chunk(const GroupedArgs &ga, int tiles, hipStream_t s)
{
    constexpr int BM = 128, BN = 128;
    const size_t lds = 2 * LdsGeo<BM, BN, 2, 2>::TILE;         // 64 KB: no attribute needed
    hipLaunchKernelGGL((grouped_prefill_kernel<BM, BN, TAIL>), dim3((unsigned)tiles), dim3(256), lds,
                       s, ga);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs *groups, int G, hipStream_t s)
{
    constexpr int BM = 128, BN = 128;
    if (G <= 0) return hipSuccess;
    const int64_t N = groups[0].N, K = groups[0].K;
    const int k = groups[0].k;
    if (N <= 0) return hipSuccess;          // K == 0 still runs: the tiles write Y = 0
    GroupedArgs ga{};
    ga.N = N;
    ga.K = K;
    ga.k = k;
    ga.tiles_n = (int)((N + BN - 1) / BN);
    for (int g0 = 0; g0 < G; g0 += GROUP_MAX) {
        const int cnt = G - g0 < GROUP_MAX ? G - g0 : GROUP_MAX;
        int tiles = 0;
        for (int i = 0; i < cnt; i++) {
            const GemmArgs &a = groups[g0 + i];
            ga.g[i] = GroupDesc{a.Xq, a.Xs, a.alpha_x, a.X_S, a.Wq, a.Ws, a.alpha_w, a.W_S, a.Y,
                                a.M > 0 ? a.M : 0};
            ga.tile_start[i] = tiles;
            tiles += (int)((ga.g[i].M + BM - 1) / BM) * ga.tiles_n;
        }
        ga.tile_start[cnt] = tiles;
        ga.G = cnt;
        if (tiles == 0) continue;
        hipError_t e = k > 0 ? launch_grouped_chunk<true>(ga, tiles, s)
                             : launch_grouped_chunk<false>(ga, tiles, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ===========================================================================
// Decode path, streaming form: a workgroup of NW waves owns CB column blocks
// (16*CB output channels) and the whole K; wave w takes K chunks (128
// channels each) w, w+NW, w+2NW, ... so the waves of a workgroup sweep each
// weight row contiguously.  Each wave keeps two batches of BB chunks of
// weight and activation codes in registers, loading one while it decodes and
// multiplies the other, so every wave has several 16-byte loads per lane in
// flight.  Partial accumulators are summed through LDS in wave order, then
// scaled, completed with the BF16 side product and stored -- one launch, no
// workspace.
// ===========================================================================
template <int MB, int CB, int NW, int BB>
struct DecodeCfg {
    static constexpr int T = MB * CB;                    // 16x16 tiles per wave
    static constexpr int RED_TILES = (T * NW <= 128) ? T : (128 / NW);   // tiles per LDS round
};

template <int MB, int CB, int NW, int BB, bool TAIL>
__device__ __forceinline__ void decode2_body(const GemmArgs &a, int64_t blk)
{
    using C = DecodeCfg<MB, CB, NW, BB>;
    __shared__ f32x4 red[NW][C::RED_TILES][WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t rowb = K / 2, rows = K / 16;
    const int64_t n0 = blk * (16 * CB);
    const int nchunk = (int)(K / BK);

    const uint8_t *wrow[CB];
    const uint8_t *wsrow[CB];
#pragma unroll
    for (int j = 0; j < CB; j++) {
        const int64_t n = n0 + j * 16 + rr;
        const int64_t nn = n < N ? n : 0;            // edge rows read row 0; never stored
        wrow[j] = a.Wq + nn * rowb + g * 16;
        wsrow[j] = a.Ws + nn * rows + 2 * g;
    }
    const uint8_t *xrow[MB];
    const uint8_t *xsrow[MB];
#pragma unroll
    for (int i = 0; i < MB; i++) {
        const int64_t m = i * 16 + rr;
        const int64_t mm = m < M ? m : 0;
        xrow[i] = a.Xq + mm * rowb + g * 16;
        xsrow[i] = a.Xs + mm * rows + 2 * g;
    }

    f32x4 acc[MB][CB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < CB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wc0[BB][CB], xc0[BB][MB], wc1[BB][CB], xc1[BB][MB];
    unsigned ws0[BB][CB], xs0[BB][MB], ws1[BB][CB], xs1[BB][MB];
    auto load = [&](int c, u32x4 (*wc)[CB], unsigned (*ws)[CB], u32x4 (*xc)[MB], unsigned (*xs)[MB]) {
#pragma unroll
        for (int b = 0; b < BB; b++) {
            const int ci = min(c + b * NW, nchunk - 1);      // clamped; masked at use
#pragma unroll
            for (int j = 0; j < CB; j++) {
                wc[b][j] = *reinterpret_cast<const u32x4 *>(wrow[j] + (int64_t)ci * CODE_ROW);
                ws[b][j] = *reinterpret_cast<const uint16_t *>(wsrow[j] + (int64_t)ci * SCALE_ROW);
            }
#pragma unroll
            for (int i = 0; i < MB; i++) {
                xc[b][i] = *reinterpret_cast<const u32x4 *>(xrow[i] + (int64_t)ci * CODE_ROW);
                xs[b][i] = *reinterpret_cast<const uint16_t *>(xsrow[i] + (int64_t)ci * SCALE_ROW);
            }
        }
    };
    auto compute = [&](int c, u32x4 (*wc)[CB], unsigned (*ws)[CB], u32x4 (*xc)[MB], unsigned (*xs)[MB]) {
#pragma unroll
        for (int b = 0; b < BB; b++) {
            const bool ok = c + b * NW < nchunk;
#pragma unroll
            for (int s = 0; s < 4; s++) {
                f16x8 af[MB];
#pragma unroll
                for (int i = 0; i < MB; i++) {
                    const unsigned code = ok ? xc[b][i][s] : 0u;
                    af[i] = decode8(code, e4m3_pair((xs[b][i] >> ((s >> 1) * 8)) & 0xFFu));
                }
#pragma unroll
                for (int j = 0; j < CB; j++) {
                    const f16x8 bf = decode8(wc[b][j][s], e4m3_pair((ws[b][j] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
                    for (int i = 0; i < MB; i++) acc[i][j] = mfma_f16(af[i], bf, acc[i][j]);
                }
            }
        }
    };

    int c = wave;
    if (c < nchunk) load(c, wc0, ws0, xc0, xs0);
    // W_S fragments (k = 32 or 64) of the tile this wave finishes, issued by
    // every wave alike right behind its first batch: the waits for later
    // batches, younger loads, include them, and by then they have arrived.
    // (Loaded in the epilogue, their HBM latency would add to the call's
    // tail.)  X_S, a few KB that every workgroup reads, comes from L2 in the
    // epilogue.  Only where each wave finishes at most one tile, in one
    // round: two would hold 8 more registers than the widest form can spare.
    constexpr int TPW = (C::T + NW - 1) / NW;
    const int k = a.k;
    const bool side_pre = TAIL && TPW == 1 && C::RED_TILES == C::T && (k == 32 || k == 64);
    bf16x8 tb[2];
    if (side_pre) {
        const int t = min(wave, C::T - 1);
        const int64_t n = n0 + (t % CB) * 16 + rr;
        const uint16_t *wb = a.W_S + (n < N ? n : 0) * k + g * 8;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int hh = (h * 32 < k) ? h : 0;              // k = 32: second half re-reads the first
            tb[h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wb + hh * 32));
        }
    }
    while (c < nchunk) {
        const int c1 = c + BB * NW;
        if (c1 < nchunk) load(c1, wc1, ws1, xc1, xs1);
        compute(c, wc0, ws0, xc0, xs0);
        if (c1 >= nchunk) break;
        const int c2 = c1 + BB * NW;
        if (c2 < nchunk) load(c2, wc0, ws0, xc0, xs0);
        compute(c1, wc1, ws1, xc1, xs1);
        c = c2;
    }

    // ---- deterministic cross-wave sum through LDS, in rounds of RED_TILES tiles
    const float alpha = (*a.alpha_x) * (*a.alpha_w);
#pragma unroll
    for (int t0 = 0; t0 < C::T; t0 += C::RED_TILES) {
        if (t0 > 0) __syncthreads();
#pragma unroll
        for (int t = 0; t < C::RED_TILES; t++)
            if (t0 + t < C::T) red[wave][t][lane] = acc[(t0 + t) / CB][(t0 + t) % CB];
        __syncthreads();
        for (int t = wave; t < C::RED_TILES && t0 + t < C::T; t += NW) {
            const int i = (t0 + t) / CB, j = (t0 + t) % CB;
            f32x4 v = red[0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; w++) v += red[w][t][lane];
            v *= alpha;
            const int64_t n = n0 + j * 16 + rr;
            const int64_t mrow = i * 16 + rr;
            if (side_pre) {                // one round, one tile per wave: t == wave
                const bf16x8 z = {};
                const bool okm = mrow < M, okn = n < N;
                const uint16_t *xa = a.X_S + (okm ? mrow : 0) * k + g * 8;
                const bf16x8 ta0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xa));
                v = mfma_bf16(okm ? ta0 : z, okn ? tb[0] : z, v);
                if (k == 64) {
                    const bf16x8 ta1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xa + 32));
                    v = mfma_bf16(okm ? ta1 : z, okn ? tb[1] : z, v);
                }
            } else if (TAIL) {
                const bool al = (k % 8) == 0;
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
}

template <int MB, int CB, int NW, int BB, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode2_kernel(GemmArgs a)
{
    decode2_body<MB, CB, NW, BB, TAIL>(a, blockIdx.x);
}

template <int MB, int CB, int NW, int BB, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode2_seg_kernel(SegTable t)
{
    int local;
    const GemmArgs a = seg_args(t, blockIdx.x, local);
    decode2_body<MB, CB, NW, BB, TAIL>(a, local);
}

template <int MB, int CB, int NW, int BB>
static hipError_t run_decode2(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, 16 * CB);
        const dim3 grid((unsigned)t.start[t.nseg]);
        if (a.k > 0)
            hipLaunchKernelGGL((decode2_seg_kernel<MB, CB, NW, BB, true>), grid, dim3(64 * NW), 0, s, t);
        else
            hipLaunchKernelGGL((decode2_seg_kernel<MB, CB, NW, BB, false>), grid, dim3(64 * NW), 0, s, t);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((a.N + 16 * CB - 1) / (16 * CB)));
    if (a.k > 0)
        hipLaunchKernelGGL((decode2_kernel<MB, CB, NW, BB, true>), grid, dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((decode2_kernel<MB, CB, NW, BB, false>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// ===========================================================================
// Decode path, single-round form.  A workgroup of NW waves owns CB column
// blocks (16*CB output channels) and the whole K; wave w owns K chunks (128
// channels each) w, w+NW, ..., at most CPW of them.  Every wave issues all of
// its weight and activation loads at once -- and, for the waves that finish
// output tiles, the BF16 side operands too -- so the kernel costs about one
// memory round trip plus the transfer itself.  Partials are summed through
// LDS in wave order, then scaled, completed with the side product and stored.
// ===========================================================================
template <int MB, int CB, int NW, int CPW, bool TAIL>
__device__ __forceinline__ void decode3_body(const GemmArgs &a, int64_t blk)
{
    constexpr int T = MB * CB;
    constexpr int RT = (T * NW <= 128) ? T : (128 / NW);      // tiles per LDS round
    __shared__ f32x4 red[NW][RT][WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);   // uniform: scalar branches
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t rowb = K / 2, rows = K / 16;
    const int64_t n0 = blk * (16 * CB);
    const int nchunk = (int)(K / BK);

    // All loads are unconditional (chunk index clamped, edge rows redirected
    // to row 0) and issued before any use; validity is applied when the data
    // is consumed, so no load waits on another.
    u32x4 wc[CPW][CB], xc[CPW][MB];
    unsigned ws[CPW][CB], xs[CPW][MB];
#pragma unroll
    for (int j = 0; j < CB; j++) {
        const int64_t n = n0 + j * 16 + rr;
        const int64_t nn = n < N ? n : 0;                      // edge rows: never stored
        const uint8_t *pw = a.Wq + nn * rowb + g * 16;
        const uint8_t *ps = a.Ws + nn * rows + 2 * g;
#pragma unroll
        for (int c = 0; c < CPW; c++) {
            const int64_t ci = min(wave + c * NW, nchunk - 1);
            wc[c][j] = *reinterpret_cast<const u32x4 *>(pw + ci * CODE_ROW);
            ws[c][j] = *reinterpret_cast<const uint16_t *>(ps + ci * SCALE_ROW);
        }
    }
#pragma unroll
    for (int i = 0; i < MB; i++) {
        const int64_t m = i * 16 + rr;
        const int64_t mm = m < M ? m : 0;                      // padding rows: never stored
        const uint8_t *px = a.Xq + mm * rowb + g * 16;
        const uint8_t *pxs = a.Xs + mm * rows + 2 * g;
#pragma unroll
        for (int c = 0; c < CPW; c++) {
            const int64_t ci = min(wave + c * NW, nchunk - 1);
            xc[c][i] = *reinterpret_cast<const u32x4 *>(px + ci * CODE_ROW);
            xs[c][i] = *reinterpret_cast<const uint16_t *>(pxs + ci * SCALE_ROW);
        }
    }
    // side operands of the tiles this wave finishes, for k = 32 or 64
    constexpr int TPW = (T + NW - 1) / NW;
    const int k = a.k;
    const bool side_pre = TAIL && (k == 32 || k == 64);
    bf16x8 ta[TPW][2], tb[TPW][2];
    if (side_pre) {
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int t = min(wave + u * NW, T - 1);
            const int i = t / CB, j = t % CB;
            const int64_t mrow = i * 16 + rr, n = n0 + j * 16 + rr;
            const uint16_t *xa = a.X_S + (mrow < M ? mrow : 0) * k + g * 8;
            const uint16_t *wb = a.W_S + (n < N ? n : 0) * k + g * 8;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int hh = (h * 32 < k) ? h : 0;          // k = 32: second half re-reads the first
                ta[u][h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xa + hh * 32));
                tb[u][h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wb + hh * 32));
            }
        }
    }

    f32x4 acc[MB][CB];
#pragma unroll
    for (int i = 0; i < MB; i++)
#pragma unroll
        for (int j = 0; j < CB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CPW; c++) {
        if (wave + c * NW < nchunk) {                          // uniform branch
#pragma unroll
            for (int s = 0; s < 4; s++) {
                f16x8 af[MB];
#pragma unroll
                for (int i = 0; i < MB; i++)
                    af[i] = decode8(xc[c][i][s], e4m3_pair((xs[c][i] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
                for (int j = 0; j < CB; j++) {
                    const f16x8 bf = decode8(wc[c][j][s], e4m3_pair((ws[c][j] >> ((s >> 1) * 8)) & 0xFFu));
#pragma unroll
                    for (int i = 0; i < MB; i++) acc[i][j] = mfma_f16(af[i], bf, acc[i][j]);
                }
            }
        }
    }

    const float alpha = (*a.alpha_x) * (*a.alpha_w);
#pragma unroll
    for (int t0 = 0; t0 < T; t0 += RT) {
        if (t0 > 0) __syncthreads();
#pragma unroll
        for (int t = 0; t < RT; t++)
            if (t0 + t < T) red[wave][t][lane] = acc[(t0 + t) / CB][(t0 + t) % CB];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < TPW; u++) {
            const int tt = wave + u * NW;                      // global tile index
            if (tt < t0 || tt >= t0 + RT || tt >= T) continue;
            const int t = tt - t0;
            const int i = tt / CB, j = tt % CB;
            f32x4 v = red[0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; w++) v += red[w][t][lane];
            v *= alpha;
            const int64_t n = n0 + j * 16 + rr;
            const int64_t mrow = i * 16 + rr;
            if (TAIL) {
                if (side_pre) {
                    const bf16x8 z = {};
                    const bool okm = mrow < M, okn = n < N;
                    v = mfma_bf16(okm ? ta[u][0] : z, okn ? tb[u][0] : z, v);
                    if (k == 64) v = mfma_bf16(okm ? ta[u][1] : z, okn ? tb[u][1] : z, v);
                } else {
                    const bool al = (k % 8) == 0;
                    for (int kk = 0; kk < k; kk += 32) {
                        const int cc = kk + g * 8;
                        const int valid = max(0, min(8, k - cc));
                        bf16x8 af = load_bf16x8(a.X_S + mrow * k + cc, (mrow < M) ? valid : 0, al);
                        bf16x8 bf = load_bf16x8(a.W_S + n * k + cc, (n < N) ? valid : 0, al);
                        v = mfma_bf16(af, bf, v);
                    }
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
}

template <int MB, int CB, int NW, int CPW, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode3_kernel(GemmArgs a)
{
    decode3_body<MB, CB, NW, CPW, TAIL>(a, blockIdx.x);
}

template <int MB, int CB, int NW, int CPW, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode3_seg_kernel(SegTable t)
{
    int local;
    const GemmArgs a = seg_args(t, blockIdx.x, local);
    decode3_body<MB, CB, NW, CPW, TAIL>(a, local);
}

// ---------------------------------------------------------------------------
// Variant for few activation rows (M*K*2 bytes fit in LDS): the workgroup
// decodes the M real activation rows once into an FP16 LDS copy, and every
// wave reads its A fragments from there instead of decoding 16 rows (most of
// them padding) per chunk.  Weight handling is the single-round scheme above.
// ---------------------------------------------------------------------------
constexpr int XLDS_MAX = 64 * 1024;        // bytes of FP16 activations kept in LDS

// SIDE: 0 for k = 0; 1 for k = 32 or 64 (side tiles staged through LDS);
// 2 for any other k (side operands loaded in the epilogue).
template <int NW, int CPW, int SIDE, int XPT>
__device__ __forceinline__ void decode_xlds_body(const GemmArgs &a, int64_t blk)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];   // [M][K] f16, then reduction space
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t rowb = K / 2, rows = K / 16;
    const int64_t n0 = blk * 16;
    const int nchunk = (int)(K / BK);

    // the thread's first XPT activation blocks (codes and scale) are loaded
    // ahead of the weights: loads complete in issue order, so the decode into
    // LDS below need not wait for the weight stream
    const int64_t nbx = K / 16;
    u32x2 xc[XPT];
    unsigned xsb[XPT];
#pragma unroll
    for (int j = 0; j < XPT; j++) {
        const int64_t it = tid + (int64_t)j * 64 * NW;
        const int64_t itc = it < M * nbx ? it : 0;
        xc[j] = *reinterpret_cast<const u32x2 *>(a.Xq + (itc / nbx) * rowb + (itc % nbx) * 8);
        xsb[j] = a.Xs[(itc / nbx) * rows + itc % nbx];
    }
    __builtin_amdgcn_sched_barrier(0);     // keep these loads ahead of the weight loads

    // weights of this wave: chunks [c0, c0 + CPW) of each of its 16 rows,
    // so the waves of the workgroup sweep every row contiguously.  Scales come
    // 16 bytes (two chunks) per load; all loads are issued before any use.
    const int c0 = wave * CPW;
    u32x4 wc[CPW];
    u32x4 wsv[CPW / 2];
    {
        const int64_t n = n0 + rr;
        const int64_t nn = n < N ? n : 0;
        const uint8_t *pw = a.Wq + nn * rowb + g * 16;
        const uint8_t *ps = a.Ws + nn * rows;
        // in the order of use: each scale pair just ahead of its two chunks
#pragma unroll
        for (int c = 0; c < CPW; c++) {
            if (c % 2 == 0) {
                const int64_t cs = min(c0 + c, nchunk - 2);
                wsv[c / 2] = *reinterpret_cast<const u32x4 *>(ps + cs * SCALE_ROW);
            }
            const int64_t ci = min(c0 + c, nchunk - 1);
            wc[c] = *reinterpret_cast<const u32x4 *>(pw + ci * CODE_ROW);
        }
    }
    // side operands for k = 32 or 64: one dword of the W_S tile (16 rows x k)
    // and one of X_S (M rows x k) per thread, so that every wave issues the
    // same loads (the compiler can then count each wave's outstanding loads
    // exactly and wait for the weights chunk by chunk); they reach wave 0,
    // which finishes the block, through LDS.  Issued after the weights: W_S
    // comes from HBM, and a wait for it ahead of the main loop (loads
    // complete in issue order) would hold the MFMAs back by its latency.
    const int k = a.k;
    const int kd = k / 2;                               // dwords per side row
    unsigned sw = 0, sx = 0;
    if (SIDE == 1) {
        const int64_t wr = min(tid / kd, 15), xr = min((int64_t)(tid / kd), M - 1);
        const int64_t n = n0 + wr;
        sw = *reinterpret_cast<const unsigned *>(a.W_S + (n < N ? n : 0) * k + (tid % kd) * 2);
        sx = *reinterpret_cast<const unsigned *>(a.X_S + xr * k + (tid % kd) * 2);
    }
    // decode the M activation rows into LDS: one 16-channel block per item
    {
        const int64_t nb = K / 16;
        auto put = [&](int64_t it, u32x2 c, unsigned sbyte) {
            const int64_t m = it / nb, b = it - m * nb;
            const f16x2 sc = e4m3_pair(sbyte);
            f16x8 *dst = reinterpret_cast<f16x8 *>(xl + (m * K + b * 16) * 2);
            dst[0] = decode8(c.x, sc);
            dst[1] = decode8(c.y, sc);
        };
#pragma unroll
        for (int j = 0; j < XPT; j++) {
            const int64_t it = tid + (int64_t)j * 64 * NW;
            if (it < M * nb) put(it, xc[j], xsb[j]);
        }
        for (int64_t it = tid + (int64_t)XPT * 64 * NW; it < M * nb; it += 64 * NW) {
            const int64_t m = it / nb, b = it - m * nb;
            put(it, *reinterpret_cast<const u32x2 *>(a.Xq + m * rowb + b * 8), a.Xs[m * rows + b]);
        }
    }
    const int64_t red_off = (M * K * 2 + 15) & ~(int64_t)15;
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool xrow = rr < M;
    const uint8_t *xbase = xl + (int64_t)(xrow ? rr : 0) * K * 2 + g * 64;   // lane's 32 channels of a chunk
#pragma unroll
    for (int c = 0; c < CPW; c++) {
        const int ci = c0 + c;
        if (ci < nchunk) {
            // scale bytes 2g, 2g+1 of chunk ci inside the 16-byte scale vector
            const int cl = min(c0 + 2 * (c / 2), nchunk - 2);           // first chunk of the vector
            const int off = (ci - cl) * 8 + 2 * g;                        // byte offset, 0..14
            const unsigned word = wsv[c / 2][off >> 2];
            const unsigned sb = (word >> ((off & 3) * 8)) & 0xFFFFu;
            const f16x2 s0 = e4m3_pair(sb & 0xFFu), s1 = e4m3_pair(sb >> 8);
#pragma unroll
            for (int s = 0; s < 4; s++) {
                f16x8 af = *reinterpret_cast<const f16x8 *>(xbase + (int64_t)ci * BK * 2 + s * 16);
                if (!xrow) af = f16x8{};
                const f16x8 bf = decode8(wc[c][s], s < 2 ? s0 : s1);
                acc = mfma_f16(af, bf, acc);
            }
        }
    }

    // wave-order reduction through LDS (reuses the space after the
    // activations); the side tiles go after it: W_S [16][kd] dwords, then
    // X_S [M][kd]
    f32x4 *red = reinterpret_cast<f32x4 *>(xl + red_off);
    uint32_t *sbuf = reinterpret_cast<uint32_t *>(xl + red_off + NW * WAVE * 16);
    red[wave * WAVE + lane] = acc;
    if (SIDE == 1) {
        if (tid < 16 * kd) sbuf[tid] = sw;
        if (tid < M * kd) sbuf[16 * kd + tid] = sx;
    }
    __syncthreads();
    if (wave == 0) {
        // the BF16 side product of the block (k = 32 or 64); lane (g, rr)
        // holds row rr, channels 32h + 8g .. +8
        f32x4 side = {0.f, 0.f, 0.f, 0.f};
        if (SIDE == 1) {
            const bf16x8 z = {};
            const bool okm = rr < M, okn = n0 + rr < N;
            const uint32_t *wrow = sbuf + rr * kd;
            const uint32_t *xrow = sbuf + 16 * kd + (okm ? rr : 0) * kd;
            for (int h = 0; h < k / 32; h++) {
                const bf16x8 ta = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xrow + 16 * h + 4 * g));
                const bf16x8 tb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wrow + 16 * h + 4 * g));
                side = mfma_bf16(okm ? ta : z, okn ? tb : z, side);
            }
        }
        f32x4 v = red[lane];
#pragma unroll
        for (int w = 1; w < NW; w++) v += red[w * WAVE + lane];
        const float alpha = (*a.alpha_x) * (*a.alpha_w);
        const int64_t n = n0 + rr;
        if (SIDE == 1) {
#pragma unroll
            for (int q = 0; q < 4; q++) v[q] = __builtin_fmaf(alpha, v[q], side[q]);
        } else {
            v *= alpha;
        }
        if (SIDE == 2) {                  // other k: direct loads, masked
            const bool al = (k % 8) == 0;
            const int64_t mrow = rr;
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
                const int64_t m = g * 4 + q;
                if (m < M) a.Y[m * a.ldy + n] = v[q];
            }
    }
}

template <int NW, int CPW, int SIDE, int XPT>
__global__ __launch_bounds__(64 * NW) void decode_xlds_kernel(GemmArgs a)
{
    decode_xlds_body<NW, CPW, SIDE, XPT>(a, blockIdx.x);
}

template <int NW, int CPW, int SIDE, int XPT>
__global__ __launch_bounds__(64 * NW) void decode_xlds_seg_kernel(SegTable t)
{
    int local;
    const GemmArgs a = seg_args(t, blockIdx.x, local);
    decode_xlds_body<NW, CPW, SIDE, XPT>(a, local);
}

template <int NW, int CPW, int SIDE, int XPT>
static hipError_t launch_xlds_x(const GemmArgs &a, const SegSpec *sp, size_t lds, hipStream_t s)
{
    constexpr int LDS_ATTR = XLDS_MAX + 16 * WAVE * 16 + 20 * 128;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_xlds_kernel<NW, CPW, SIDE, XPT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS_ATTR);
    static const hipError_t attr_seg = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_xlds_seg_kernel<NW, CPW, SIDE, XPT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS_ATTR);
    if (attr != hipSuccess) return attr;
    if (attr_seg != hipSuccess) return attr_seg;
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, 16);
        hipLaunchKernelGGL((decode_xlds_seg_kernel<NW, CPW, SIDE, XPT>), dim3((unsigned)t.start[t.nseg]),
                           dim3(64 * NW), lds, s, t);
    } else {
        hipLaunchKernelGGL((decode_xlds_kernel<NW, CPW, SIDE, XPT>), dim3((unsigned)((a.N + 15) / 16)),
                           dim3(64 * NW), lds, s, a);
    }
    return hipGetLastError();
}

// activation blocks per thread loaded ahead of the weights: all of them when
// they are at most two per thread (the rest, if any, behind the weights)
template <int NW, int CPW, int SIDE>
static hipError_t launch_xlds(const GemmArgs &a, const SegSpec *sp, size_t lds, hipStream_t s)
{
    if (a.M * a.K / 16 <= 64 * NW) return launch_xlds_x<NW, CPW, SIDE, 1>(a, sp, lds, s);
    return launch_xlds_x<NW, CPW, SIDE, 2>(a, sp, lds, s);
}

template <int NW, int CPW>
static hipError_t run_decode_xlds(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    // activations, reduction space, side tiles (k <= 64: (16 + M) rows of 128 bytes)
    const size_t lds = (size_t)((a.M * a.K * 2 + 15) & ~(int64_t)15) + (size_t)NW * WAVE * 16 +
                       (a.k > 0 ? (size_t)(16 + a.M) * 128 : 0);
    if (a.k == 32 || a.k == 64) return launch_xlds<NW, CPW, 1>(a, sp, lds, s);
    if (a.k > 0) return launch_xlds<NW, CPW, 2>(a, sp, lds, s);
    return launch_xlds<NW, CPW, 0>(a, sp, lds, s);
}

template <int MB, int CB, int NW, int CPW>
static hipError_t run_decode3(const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, 16 * CB);
        const dim3 grid((unsigned)t.start[t.nseg]);
        if (a.k > 0)
            hipLaunchKernelGGL((decode3_seg_kernel<MB, CB, NW, CPW, true>), grid, dim3(64 * NW), 0, s, t);
        else
            hipLaunchKernelGGL((decode3_seg_kernel<MB, CB, NW, CPW, false>), grid, dim3(64 * NW), 0, s, t);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((a.N + 16 * CB - 1) / (16 * CB)));
    if (a.k > 0)
        hipLaunchKernelGGL((decode3_kernel<MB, CB, NW, CPW, true>), grid, dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((decode3_kernel<MB, CB, NW, CPW, false>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// waves per workgroup so that each wave holds at most CPW chunks; false when
// even MAXNW waves would need more (then the looping form is used)
template <int MB, int CB, int CPW, int MAXNW>
static bool run_decode3_k(const GemmArgs &a, const SegSpec *sp, hipStream_t s, hipError_t &e)
{
    const int nchunk = (int)(a.K / BK);
    if (nchunk <= 4 * CPW) { e = run_decode3<MB, CB, 4, CPW>(a, sp, s); return true; }
    if (nchunk <= 8 * CPW) { e = run_decode3<MB, CB, 8, CPW>(a, sp, s); return true; }
    if (MAXNW >= 16 && nchunk <= 16 * CPW) { e = run_decode3<MB, CB, (MAXNW >= 16 ? 16 : 8), CPW>(a, sp, s); return true; }
    return false;
}

// ===========================================================================
size_t gemm_ws_bytes(Path, int64_t, int64_t, int64_t)
{
    return 0;        // neither datapath needs scratch memory
}

// configuration choice and launch; sp != nullptr: the column segments of sp,
// whose widths sum to a.N
static hipError_t dispatch_gemm(Path p, const GemmArgs &a, const SegSpec *sp, hipStream_t s)
{
    if (a.M == 0 || a.N == 0) return hipSuccess;
    if (a.K == 0) p = Path::Prefill;    // the decode kernels assume at least one K chunk
    if (p == Path::Prefill) {
        // largest tile that still gives every CU a tile
        const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
        const int64_t t256x128 = ((a.M + 255) / 256) * ((a.N + 127) / 128);
        (void)t256x128;
        if (t256 >= 240) return a.k > 0 ? launch_prefill_lds<true>(a, sp, s) : launch_prefill_lds<false>(a, sp, s);
        return a.k > 0 ? launch_prefill_lds128<true>(a, sp, s) : launch_prefill_lds128<false>(a, sp, s);
    }
    // weight-streaming decode path; configurations chosen from measured sweeps
    // on MI355X (Qwen3-8B projection shapes, M = 1, 4, 8, 16, 32, 64)
    hipError_t e = hipSuccess;
    const int nchunk = (int)(a.K / BK);
    const int64_t colblocks = (a.N + 15) / 16;
    if (a.M <= 16) {
        if (a.M <= 4 && a.M * a.K * 2 <= XLDS_MAX && nchunk >= 2 && nchunk % 2 == 0) {   // 16-byte aligned scale pairs
            if (nchunk <= 8 * 4) return run_decode_xlds<8, 4>(a, sp, s);
            if (nchunk <= 16 * 4) return run_decode_xlds<16, 4>(a, sp, s);
            if (nchunk <= 16 * 6) return run_decode_xlds<16, 6>(a, sp, s);
            if (nchunk <= 16 * 8) return run_decode_xlds<16, 8>(a, sp, s);
        }
        // wide N: 48 columns per workgroup, streaming one chunk at a time
        // (N = 12288: 6-9% faster than the single-round form at M = 8-16);
        // K up to 4096: single round, eight waves of four chunks; longer K:
        // streaming, 16 columns per workgroup (K = 12288: 25% faster than the
        // single round at M = 4-16, whose sixteen waves hold six chunks each)
        if (colblocks >= 512) return run_decode2<1, 3, 8, 1>(a, sp, s);
        if (nchunk <= 32) return run_decode3<1, 1, 8, 4>(a, sp, s);
        return run_decode2<1, 1, 8, 1>(a, sp, s);
    }
    // M in 17..64: wide N at M <= 32 takes the single-round form with 48
    // columns per workgroup (one workgroup per CU at N = 12288); otherwise
    // the streaming form over 8 waves
    if (a.M <= 32) {
        if (colblocks >= 512 && run_decode3_k<2, 3, 4, 8>(a, sp, s, e)) return e;
        return run_decode2<2, 1, 8, 1>(a, sp, s);
    }
    if (colblocks >= 512) return run_decode2<4, 3, 8, 1>(a, sp, s);
    return run_decode2<4, 1, 8, 2>(a, sp, s);
}

hipError_t launch_gemm(Path p, const GemmArgs &a, void *, size_t, hipStream_t s)
{
    return dispatch_gemm(p, a, nullptr, s);
}

hipError_t launch_gemm_seg(Path p, const GemmArgs &a, const GemmSeg *seg, int nseg, hipStream_t s)
{
    // the configuration is chosen for the combined width, as for one call
    // with N = the sum of the widths
    GemmArgs b = a;
    b.N = 0;
    for (int i = 0; i < nseg; i++) b.N += seg[i].N;
    if (nseg == 0 || b.M == 0 || b.N == 0) return hipSuccess;
    const SegSpec sp{seg, nseg};
    return dispatch_gemm(p, b, &sp, s);
}

}  // namespace splice
