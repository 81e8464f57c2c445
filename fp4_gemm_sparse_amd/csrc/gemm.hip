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
#include "../../include/splice.h"
#include "common.hpp"
#include "kernels.hpp"
#include "segments.hpp"

#include <algorithm>

namespace splice {

constexpr int BK = 128;              // channels per decode-path K chunk
constexpr int CODE_ROW = BK / 2;     // 64 code bytes per row per chunk
constexpr int SCALE_ROW = BK / 16;   // 8 scale bytes per row per chunk
constexpr int DECODE_SPLIT_MAX = 8;  // K splits of a decode-path column group at most

// ===========================================================================
// Prefill path
// ===========================================================================
// XCD-aware tile order: consecutive workgroups go to different XCDs round
// robin, so each XCD is handed a contiguous range of work items; inside it
// tiles walk GM tile-rows at a time so neighbours share operand rows in L2.
__device__ __forceinline__ int xcd_order(int wg, int nwg)
{
    const int q = nwg / 8, r = nwg % 8;
    const int x = wg % 8, local = wg / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

__device__ __forceinline__ void group_tile(int tile, int tiles_m, int tiles_n, int &tm, int &tn)
{
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in = tile - group * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

__device__ __forceinline__ void tile_of(int wg, int nwg, int tiles_m, int tiles_n, int &tm, int &tn)
{
    group_tile(xcd_order(wg, nwg), tiles_m, tiles_n, tm, tn);
}

// with the K range split nsplit ways: the splits of a tile are consecutive
// work items, so they usually run side by side on one XCD
__device__ __forceinline__ void tile_split_of(int wg, int nwg, int nsplit, int tiles_m, int tiles_n,
                                              int &tm, int &tn, int &split)
{
    const int item = xcd_order(wg, nwg);
    const int tile = item / nsplit;
    split = item - tile * nsplit;
    group_tile(tile, tiles_m, tiles_n, tm, tn);
}

// K split over workgroups: the workgroups of one output tile each sum a range
// of K steps; the partial tiles go to the workspace and the workgroup that
// completes the tile's arrival count adds them in split order and finishes the
// tile.  wtile numbers the tile's counter and partial slots.
struct SplitK {
    int split = 0, nsplit = 1;
    int64_t wtile = 0;
    unsigned *cnt = nullptr;
    float *part = nullptr;
};

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
// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled at compile time
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

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
// PF: register stages of operand codes in flight.  The codes of step t are
// loaded PF steps ahead (at the end of step t - 1 - PF) and decoded during
// step t - 1, so a load has PF - 1 full steps of matrix work to arrive; with
// PF = 1 it is issued just before the barrier that precedes its use and the
// first decode of the next step waits for it.  The scale bytes are held as
// 16-bit values (widened to 32 bits, the compiler masked them at the loop's
// back edge, which waited for the stages just issued).
// SPLIT: the kernel may split K over workgroups (sk.nsplit > 1); only then is
// the partial-tile epilogue compiled in.
template <int BM, int BN, int WGM, int WGN, bool TAIL, int PF = 1, bool SPLIT = false>
__device__ __forceinline__ void lds_tile(const GemmArgs &a, int tm, int tn, uint8_t *lds,
                                         const SplitK &sk = SplitK{})
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
    // this workgroup's K steps [kt0, kt0 + nk) of 64 channels
    const int nk_all = (int)(K / C::BKL);
    const int nsplit = SPLIT ? sk.nsplit : 1;
    const int per_split = (nk_all + nsplit - 1) / nsplit;
    const int kt0 = SPLIT ? sk.split * per_split : 0;
    const int nk = max(0, min(nk_all - kt0, per_split));

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
    // register stage r holds the codes of the steps t with t % PF == r
    u32x4 pc[PF][UNITS];
    uint16_t ps[PF][UNITS];
    auto gload = [&](int r, int kt) {
#pragma unroll
        for (int i = 0; i < UNITS; i++) {
            pc[r][i] = *reinterpret_cast<const u32x4 *>(ucode[i] + (int64_t)kt * 32);
            ps[r][i] = *reinterpret_cast<const uint16_t *>(uscale[i] + (int64_t)kt * 4);
        }
    };
    // piece d (8 channels) of every unit of stage r into `tile`
    auto decode_piece = [&](uint8_t *tile, int r, int d) {
#pragma unroll
        for (int i = 0; i < UNITS; i++) {
            const f16x2 sc = e4m3_pair(d < 2 ? (ps[r][i] & 0xFFu) : ((ps[r][i] >> 8) & 0xFFu));
            *reinterpret_cast<f16x8 *>(tile + f16_off(urow[i], half * 4 + d)) = decode8(pc[r][i][d], sc);
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
#pragma unroll
        for (int r = 0; r < PF; r++) gload(r, kt0 + min(r, nk - 1));
#pragma unroll
        for (int d = 0; d < 4; d++) decode_piece(lds, 0, d);
        gload(0, kt0 + min(PF, nk - 1));
    }
    __syncthreads();
    const int arow = wm * C::WM + rr, brow = C::BM + wn * C::WN + rr;
    // The main loop for a wave whose first FMV 32-row fragments hold rows
    // inside M: it reads and multiplies only those (the others would only feed
    // outputs that are never stored).  FMV = FM everywhere but in the last
    // tile row of a product whose M is not a multiple of the tile; each count
    // is its own branch-free copy of the loop.
    auto main_loop = [&](auto fmv) {
    constexpr int FMV = decltype(fmv)::value;
    // K step kt; its decode fills register stage (u + 1) % PF's step into
    // the idle buffer, and the stage is refilled PF steps ahead
    auto step = [&](int kt, auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int rs = (u + 1) % PF;     // stage holding step kt + 1
        const uint8_t *cur = lds + (kt & 1) * C::TILE;
        uint8_t *nxt = lds + ((kt + 1) & 1) * C::TILE;
        f16x8 a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
#pragma unroll
        for (int i = 0; i < FMV; i++) a0[i] = *reinterpret_cast<const f16x8 *>(cur + f16_off(arow + i * 32, g));
#pragma unroll
        for (int j = 0; j < C::FN; j++) b0[j] = *reinterpret_cast<const f16x8 *>(cur + f16_off(brow + j * 32, g));
#pragma unroll
        for (int s = 0; s < 4; s++) {
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < FMV; i++)
                    a1[i] = *reinterpret_cast<const f16x8 *>(cur + f16_off(arow + i * 32, (s + 1) * 2 + g));
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    b1[j] = *reinterpret_cast<const f16x8 *>(cur + f16_off(brow + j * 32, (s + 1) * 2 + g));
            }
            decode_piece(nxt, rs, s);     // on the last step this fills the idle buffer
#pragma unroll
            for (int j = 0; j < C::FN; j++)
#pragma unroll
                for (int i = 0; i < FMV; i++) acc[i][j] = mfma32_f16(a0[i], b0[j], acc[i][j]);
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < FMV; i++) a0[i] = a1[i];
#pragma unroll
                for (int j = 0; j < C::FN; j++) b0[j] = b1[j];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        gload(rs, kt0 + min(kt + 1 + PF, nk - 1));
        lds_barrier();      // the prefetches of steps kt+2 .. kt+1+PF stay in flight
    };
    // Whole groups of PF steps in the loop, the rest after it: a loop body
    // with no exit between its steps lets the compiler see that each step
    // waits only for the stage loaded PF steps earlier (with exits inside the
    // body it waited for every load in flight at the top of each group, the
    // ones just issued included).
    int kt = 0;
    for (; kt + PF <= nk; kt += PF)
        static_for<PF>([&](auto uc) { step(kt + decltype(uc)::value, uc); });
    static_for<PF - 1>([&](auto uc) {
        if (kt + decltype(uc)::value < nk) step(kt + decltype(uc)::value, uc);
    });
    };
    // valid fragment rows of this wave (wave-uniform)
    const int fm_ok = (int)min<int64_t>(C::FM, max<int64_t>(0, (M - (m0 + wm * C::WM) + 31) / 32));
    static_assert(C::FM == 1 || C::FM == 2 || C::FM == 4, "fragment rows per wave");
    if (fm_ok >= C::FM)
        main_loop(std::integral_constant<int, C::FM>{});
    else if (fm_ok == 0)
        main_loop(std::integral_constant<int, 0>{});
    else if (fm_ok == 1)
        main_loop(std::integral_constant<int, 1>{});
    else if constexpr (C::FM == 4) {
        if (fm_ok == 2)
            main_loop(std::integral_constant<int, 2>{});
        else
            main_loop(std::integral_constant<int, 3>{});
    }

    // ---- K split over workgroups: the partial tile goes to the workspace with
    // device-coherent 8-byte stores (they bypass the non-coherent caches, so no
    // cache needs flushing); once every wave's stores have completed, one
    // thread counts the workgroup in.  The workgroup that completes the count
    // reads every split's partial with device-coherent loads, sums them in
    // split order and finishes the tile; it returns the count to zero.
    // Side operands of the epilogue (k a multiple of 16): staged through the
    // idle LDS stage buffers, 64 channels per buffer, in the tile's swizzled
    // 128-byte-row layout.  Thread (r0, cc) moves chunk cc of rows r0 + RS*u;
    // rows past M or N are clamped and channels past k re-read the last ones
    // (neither reaches a stored output).
    const int k = TAIL ? a.k : 0;
    const bool staged = TAIL && k > 0 && k % 16 == 0;
    const int kn0 = staged ? min(2 * C::BKL, k) : 0;      // channels of the first pass
    constexpr int RS = NT / 8, PU = C::ROWS * 8 / NT;
    auto stage_load = [&](int kp, int ch, u32x4 (&v)[PU]) {
        const int r0 = tid >> 3, cc = tid & 7;
        const uint16_t *xp = a.X_S + cc * 8, *wp = a.W_S + cc * 8;
        const int c = min(kp + ch * C::BKL + cc * 8, k - 8) - cc * 8;
#pragma unroll
        for (int u = 0; u < PU; u++) {
            const int row = r0 + RS * u;
            v[u] = row < C::BM ? *reinterpret_cast<const u32x4 *>(xp + min(m0 + row, M - 1) * k + c)
                               : *reinterpret_cast<const u32x4 *>(wp + min(n0 + row - C::BM, N - 1) * k + c);
        }
    };
    auto stage_store = [&](int ch, const u32x4 (&v)[PU]) {
        const int r0 = tid >> 3, cc = tid & 7;
#pragma unroll
        for (int u = 0; u < PU; u++)
            *reinterpret_cast<u32x4 *>(lds + ch * C::TILE + f16_off(r0 + RS * u, cc)) = v[u];
    };
    auto stage = [&](int kp, int kn) {              // all loads of a buffer before its stores
        for (int ch = 0; ch * C::BKL < kn; ch++) {
            u32x4 v[PU];
            stage_load(kp, ch, v);
            stage_store(ch, v);
        }
        lds_barrier();
    };
    bool first_staged = false;
    // K split, up to 64 side channels: the finishing workgroup loads each
    // wave's side fragments straight into registers ahead of the partial
    // tiles, so neither an LDS staging pass nor its barrier sits in the
    // launch's serial tail; the products are summed in the staged order
    bool side_direct = false;
    bf16x8 sxa[SPLIT ? C::FM : 1][4], swb[SPLIT ? C::FN : 1][4];

    if (SPLIT && sk.nsplit > 1) {
        __shared__ int last_flag;
        constexpr int NWV = NT / WAVE;
        // a wave's partial tile: FM x FN fragments of four 16-byte pieces per
        // lane, each piece stored lane-contiguous (one 1 KB row per wave)
        constexpr int PV = C::FM * C::FN * 4;
        constexpr uint32_t SPLIT_BYTES = (uint32_t)C::BM * C::BN * 4;
        const __amdgpu_buffer_rsrc_t rs =
            coherent_rsrc(sk.part + sk.wtile * (int64_t)sk.nsplit * (C::BM * C::BN), sk.nsplit * SPLIT_BYTES);
        auto off = [&](int sp, int pv) -> uint32_t {
            return (uint32_t)sp * SPLIT_BYTES + (uint32_t)(((wave * PV + pv) * WAVE + lane) * 16);
        };
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int j = 0; j < C::FN; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    coherent_store16(rs, off(sk.split, (i * C::FN + j) * 4 + q), __builtin_bit_cast(u32x4, v));
                }
        wait_vmem();
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(sk.cnt + sk.wtile, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            const bool last = prev == (unsigned)(sk.nsplit - 1);
            if (last) __hip_atomic_store(sk.cnt + sk.wtile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = last;
        }
        __syncthreads();
        if (!last_flag) return;
        // the first 64 side channels are loaded before the partial tiles, so
        // their latency passes while the partials arrive (loads complete in
        // issue order: the partials' waits cover them)
        u32x4 pre[PU];
        side_direct = staged && k <= 64;
        if (side_direct) {
            // rows past M or N read the last row (clamped) and are zeroed
            const bf16x8 z = {};
#pragma unroll
            for (int i = 0; i < C::FM; i++) {
                const int64_t m = m0 + wm * C::WM + i * 32 + rr;
                const uint16_t *xp = a.X_S + min<int64_t>(m, M - 1) * k + g * 8;
#pragma unroll
                for (int kk = 0; kk < 4; kk++) {
                    const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(xp + min(kk * 16, k - 16)));
                    sxa[SPLIT ? i : 0][kk] = m < M ? v : z;
                }
            }
#pragma unroll
            for (int j = 0; j < C::FN; j++) {
                const int64_t n = n0 + wn * C::WN + j * 32 + rr;
                const uint16_t *wp = a.W_S + min<int64_t>(n, N - 1) * k + g * 8;
#pragma unroll
                for (int kk = 0; kk < 4; kk++) {
                    const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wp + min(kk * 16, k - 16)));
                    swb[SPLIT ? j : 0][kk] = n < N ? v : z;
                }
            }
            first_staged = true;          // nothing left to stage for the first pass
        } else if (staged) {
            stage_load(0, 0, pre);
        }
        // The partial tiles are read two splits deep: split sp + 1's loads are
        // issued before split sp is added.  (Because the later loads are
        // conditional, the compiler's wait before each add after the first
        // also covers the loads just issued; a single-exit form without that
        // wait, measured together with the side product computed ahead of the
        // sums, was slower.)  The sum runs in split order.
        u32x4 pbuf[2][PV];
        auto pload = [&](int sp, u32x4 (&b)[PV]) {
#pragma unroll
            for (int pv = 0; pv < PV; pv++) b[pv] = coherent_load16(rs, off(sp, pv));
            __builtin_amdgcn_sched_barrier(0);
        };
        auto padd = [&](const u32x4 (&b)[PV], bool first) {
#pragma unroll
            for (int i = 0; i < C::FM; i++)
#pragma unroll
                for (int j = 0; j < C::FN; j++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const f32x4 t = __builtin_bit_cast(f32x4, b[(i * C::FN + j) * 4 + q]);
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            acc[i][j][4 * q + e] = first ? t[e] : acc[i][j][4 * q + e] + t[e];
                    }
        };
        pload(0, pbuf[0]);
        for (int sp = 0; sp < sk.nsplit; sp += 2) {
            if (sp + 1 < sk.nsplit) pload(sp + 1, pbuf[1]);
            padd(pbuf[0], sp == 0);
            if (sp + 1 >= sk.nsplit) break;
            if (sp + 2 < sk.nsplit) pload(sp + 2, pbuf[0]);
            padd(pbuf[1], false);
        }
        if (staged && !side_direct) {
            stage_store(0, pre);
            if (kn0 > C::BKL) {
                u32x4 v[PU];
                stage_load(0, 1, v);
                stage_store(1, v);
            }
            lds_barrier();
            first_staged = true;
        }
    }

    // ---- epilogue: Y = alpha_x*alpha_w * acc + X_S W_S^T
    // The side operands (k a multiple of 16) go through the LDS stage buffers
    // (stage above) in passes of up to 128 channels.  Per 32-row fragment the
    // side product goes into a small separate accumulator and the first pass
    // stores Y = fma(alpha, acc, side), so the FP4 accumulator is only read;
    // further passes (k > 128) add their side products into Y.
    const float alpha = (*a.alpha_x) * (*a.alpha_w);
    const int64_t mb = m0 + wm * C::WM + g * 4, nb = n0 + wn * C::WN + rr;
    float *yb = a.Y + mb * a.ldy + nb;
    const bool full = m0 + C::BM <= M && n0 + C::BN <= N;
    // The first store of Y is non-temporal: the output is not read again by
    // this launch, and every CU ends its tile at about the same time, so the
    // burst drains without taking L2 lines from the next tiles' operands
    // (gate at M = 8192: 2% faster).  Later passes (k > 128) read Y back.
    auto put = [&](float *y, float v, bool add) {
        if (add)
            *y = *y + v;
        else
            __builtin_nontemporal_store(v, y);
    };
    auto store_rows = [&](int i, const f32x16 (&v)[C::FN], bool add) {
        if (full) {
#pragma unroll
            for (int q = 0; q < 16; q++) {
                float *yr = yb + (int64_t)(i * 32 + (q >> 2) * 8 + (q & 3)) * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++) put(yr + j * 32, v[j][q], add);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int dm = i * 32 + (q >> 2) * 8 + (q & 3);
                if (mb + dm >= M) continue;
                float *yr = yb + (int64_t)dm * a.ldy;
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    if (nb + j * 32 < N) put(yr + j * 32, v[j][q], add);
            }
        }
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
    if (staged && !first_staged) stage(0, kn0);
#pragma unroll
    for (int i = 0; i < C::FM; i++) {
        f32x16 side[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; j++)
#pragma unroll
            for (int q = 0; q < 16; q++) side[j][q] = 0.f;
        if (SPLIT && side_direct) {
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
                if (kk < k / 16)
#pragma unroll
                    for (int j = 0; j < C::FN; j++)
                        side[j] = mfma32_bf16(sxa[SPLIT ? i : 0][kk], swb[SPLIT ? j : 0][kk], side[j]);
        } else if (staged) {
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

// code stages in flight for the 256 x 256 tile: two (2.1-3.0% faster than
// one on q, gate and down at M = 8192; three measured the same as two)
constexpr int PF256 = 2;

template <bool TAIL>
__global__ __launch_bounds__(512) void prefill_lds_kernel(GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((a.M + 255) / 256), tiles_n = (int)((a.N + 255) / 256);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    lds_tile<256, 256, 2, 4, TAIL, PF256>(a, tm, tn, lds);
}

// code stages in flight for the 128 x 128 tile (one wave per SIMD per
// workgroup): three measured 5-9% faster than one at M = 65..1024
constexpr int PF128 = 3;
// the same tile with the K range split over workgroups runs at most 256
// workgroups, one per CU, so a lane may hold up to 512 registers.  Ranges of
// more than 16 K steps keep six steps of codes in flight, shorter ones three
// (measured on MI355X, us, three / six stages: q at M = 128 in eight ranges
// of 8 steps 23.5 / 24.3, k 20.4 / 21.4; down at M = 128 in eight of 24
// steps 37.1 / 36.6, at M = 256 in four of 48 50.2 / 48.5; gate at M = 65 in
// two of 32 35.9 / 35.0).
constexpr int PF128S_SHORT = 3, PF128S_LONG = 6, PF128S_SHORT_MAX_STEPS = 16;

// 128 x 128 tiles, four waves of 64 x 64: for grids too small for the
// 256 x 256 tile.  Unsplit, two workgroups per CU (so at most 256 registers
// per lane: the launch bound says so).  Where even these tiles leave CUs
// idle, the K range is split nsplit ways (cnt and part in the workspace),
// one workgroup per CU; only these instances compile the split epilogue.
template <bool TAIL, int PF, int OCC>
__global__ __launch_bounds__(256, OCC) void prefill_lds128_kernel(GemmArgs a, int nsplit, unsigned *cnt, float *part)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((a.M + 127) / 128), tiles_n = (int)((a.N + 127) / 128);
    int tm, tn, split;
    tile_split_of(blockIdx.x, gridDim.x, nsplit, tiles_m, tiles_n, tm, tn, split);
    SplitK sk;
    sk.split = split;
    sk.nsplit = nsplit;
    sk.wtile = (int64_t)tm * tiles_n + tn;
    sk.cnt = cnt;
    sk.part = part;
    lds_tile<128, 128, 2, 2, TAIL, PF, OCC == 1>(a, tm, tn, lds, sk);
}

// the same tiles over column segments: tile columns numbered across them
template <int BT, int WGN, bool TAIL, int PF, int OCC>
__global__ __launch_bounds__(64 * 2 * WGN, OCC) void prefill_seg_kernel(SegTable t, int nsplit, unsigned *cnt,
                                                                   float *part)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((t.a.M + BT - 1) / BT), tiles_n = t.start[t.nseg];
    int tm, tn, local, split;
    tile_split_of(blockIdx.x, gridDim.x, nsplit, tiles_m, tiles_n, tm, tn, split);
    const GemmArgs a = seg_args(t, tn, local);
    SplitK sk;
    sk.split = split;
    sk.nsplit = nsplit;
    sk.wtile = (int64_t)tm * tiles_n + tn;
    sk.cnt = cnt;
    sk.part = part;
    lds_tile<BT, BT, 2, WGN, TAIL, PF, (BT == 128 && OCC == 1)>(a, tm, local, lds, sk);
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

// Groups of at most GROUP_SMALL_M rows take 64 x 192 tiles (four waves of
// 32 x 96, the same 256 LDS rows per step as 128 x 128): a small group's
// 128 x 128 tiles decoded 128 activation rows for at most 64 real ones, and
// sixteen of them per 2048 columns against eleven.
constexpr int GROUP_SMALL_M = 64, GROUP_SMALL_BN = 192;

template <int BM, int BN, bool TAIL>
__global__ __launch_bounds__(256, 2) void grouped_prefill_kernel(GroupedArgs ga)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int w = blockIdx.x;
    int e = 0;
    while (e + 1 < ga.G && w >= ga.tile_start[e + 1]) e++;
    const int local = w - ga.tile_start[e];
    const GroupDesc &d = ga.g[e];
    const GemmArgs a{d.Xq, d.Xs, d.alpha_x, d.X_S, d.Wq, d.Ws, d.alpha_w, d.W_S,
                     d.M, ga.N, ga.K, ga.k, d.Y, ga.N};
    if (d.M <= GROUP_SMALL_M)
        lds_tile<GROUP_SMALL_M, GROUP_SMALL_BN, 2, 2, TAIL, PF128>(a, 0, local, lds);
    else
        lds_tile<BM, BN, 2, 2, TAIL, PF128>(a, local / ga.tiles_n, local % ga.tiles_n, lds);
}

// ---------------------------------------------------------------------------
// Prefill plan: the 256 x 256 tile when its grid fills the GPU or the
// 128 x 128 grid needs more than one round, else the 128 x 128 tile.  At up
// to 128 tiles the K range is also split, as many ways as keep the
// workgroups within 256 (one per CU) and each split at least eight 64-channel
// steps: at M = 65..1024 on the Qwen3-8B shapes that count was the
// fastest measured or within 1 us of it (q at M = 128: 52 us unsplit, 27 us in
// eight splits; q at M = 512, 128 tiles: 51.5 -> 37.4 us in two; down at
// M = 256: 145 -> 52 us in four).  More workgroups than CUs measured slower
// (gate at M = 65, 96 tiles: 37 us in two splits, 48 us in three; 192 tiles
// unsplit 55 us, in two 68 us).  The partial tiles take at most 256 x 64 KB.
struct PrefillPlan {
    bool big;
    int nsplit;
    int64_t tiles;     // output tiles (of the chosen size)
    size_t ws;         // workspace: tile counters, then nsplit partial tiles each
};

// The arrival counters sit in a fixed region at the front of the workspace,
// one slot per output tile, whatever the shape: splits happen only below
// SPLIT_MAX_TILES tiles, so a call never reads another shape's partial tiles
// as counters, and every call leaves all of them zero.
constexpr int64_t SPLIT_MAX_TILES = 128;
constexpr int64_t SPLIT_WORKGROUPS = 256;     // tiles x splits at most
constexpr int64_t SPLIT_MIN_STEPS = 8;        // 64-channel K steps per split at least
static_assert(SPLIT_MAX_TILES * 4 <= (int64_t)SPLIT_COUNTER_BYTES, "counter region");
// the largest workspace any shape takes fits the allocation-free entry's array
static_assert(SPLIT_COUNTER_BYTES + (size_t)SPLIT_WORKGROUPS * 128 * 128 * 4 <= SPLICE_NOALLOC_SCRATCH_BYTES,
              "no-alloc scratch");

// tiles_n128: tile columns at 128 (the segment launch counts them per segment)
static PrefillPlan plan_prefill(int64_t M, int64_t N, int64_t K, int64_t tiles_n128)
{
    PrefillPlan p{false, 1, 0, 0};
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * tiles_n128;
    // the 256 x 256 tile when its grid fills the GPU, or when the 128 x 128
    // tiles need more than one round at two per CU: a round of 256 x 256
    // tiles (one per CU) takes about 4/3 of a full 128 x 128 round, so one
    // big round beats one and a bit small ones (gate at M = 1024: 128 against
    // 162 us; a gate shard of 1536 columns at M = 8192: 121 against 165 us),
    // while at most one small round is as fast or faster (q at M = 2048: 107
    // against 109 us; q at M = 1536: 101 against 86 us)
    if (t256 >= 240 || t128 > 512) {
        p.big = true;
        p.tiles = t256;
        return p;
    }
    p.tiles = t128;
    const int64_t nk = K / LdsCfg::BKL;
    if (p.tiles <= SPLIT_MAX_TILES && p.tiles > 0) {
        int64_t sp = std::min<int64_t>(SPLIT_WORKGROUPS / p.tiles, nk / SPLIT_MIN_STEPS);
        if (sp > 1) {
            const int64_t per = (nk + sp - 1) / sp;
            sp = (nk + per - 1) / per;          // every split holds at least one step
        }
        p.nsplit = (int)std::max<int64_t>(sp, 1);
    }
    if (p.nsplit > 1) p.ws = SPLIT_COUNTER_BYTES + (size_t)p.tiles * p.nsplit * 128 * 128 * 4;
    return p;
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
        reinterpret_cast<const void *>(&prefill_seg_kernel<256, 4, TAIL, PF256, 1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    if (attr_seg != hipSuccess) return attr_seg;
    const int64_t tiles_m = (a.M + C::BM - 1) / C::BM;
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, C::BN);
        hipLaunchKernelGGL((prefill_seg_kernel<256, 4, TAIL, PF256, 1>), dim3((unsigned)(tiles_m * t.start[t.nseg])),
                           dim3(C::NT), lds, s, t, 1, (unsigned *)nullptr, (float *)nullptr);
    } else {
        const int64_t tiles = tiles_m * ((a.N + C::BN - 1) / C::BN);
        hipLaunchKernelGGL(prefill_lds_kernel<TAIL>, dim3((unsigned)tiles), dim3(C::NT), lds, s, a);
    }
    return hipGetLastError();
}

template <bool TAIL>
static hipError_t launch_prefill_lds128(const GemmArgs &a, const SegSpec *sp, const PrefillPlan &p, void *ws,
                                        hipStream_t s)
{
    using C = LdsGeo<128, 128, 2, 2>;
    const size_t lds = 2 * C::TILE;
    unsigned *cnt = p.nsplit > 1 ? static_cast<unsigned *>(ws) : nullptr;
    float *part = p.nsplit > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + SPLIT_COUNTER_BYTES)
                               : nullptr;
    const dim3 grid((unsigned)(p.tiles * p.nsplit));
    const int64_t nk = a.K / LdsCfg::BKL;
    const bool long_range = p.nsplit > 1 && (nk + p.nsplit - 1) / p.nsplit > PF128S_SHORT_MAX_STEPS;
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, C::BN);
        if (p.nsplit == 1)
            hipLaunchKernelGGL((prefill_seg_kernel<128, 2, TAIL, PF128, 2>), grid, dim3(C::NT), lds, s, t, p.nsplit,
                               cnt, part);
        else if (long_range)
            hipLaunchKernelGGL((prefill_seg_kernel<128, 2, TAIL, PF128S_LONG, 1>), grid, dim3(C::NT), lds, s, t,
                               p.nsplit, cnt, part);
        else
            hipLaunchKernelGGL((prefill_seg_kernel<128, 2, TAIL, PF128S_SHORT, 1>), grid, dim3(C::NT), lds, s, t,
                               p.nsplit, cnt, part);
    } else {
        if (p.nsplit == 1)
            hipLaunchKernelGGL((prefill_lds128_kernel<TAIL, PF128, 2>), grid, dim3(C::NT), lds, s, a, p.nsplit, cnt,
                               part);
        else if (long_range)
            hipLaunchKernelGGL((prefill_lds128_kernel<TAIL, PF128S_LONG, 1>), grid, dim3(C::NT), lds, s, a, p.nsplit,
                               cnt, part);
        else
            hipLaunchKernelGGL((prefill_lds128_kernel<TAIL, PF128S_SHORT, 1>), grid, dim3(C::NT), lds, s, a, p.nsplit,
                               cnt, part);
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
        // the largest groups' tiles first: workgroups are dispatched in
        // order, so the cheaper tiles of the small groups fill the last round
        int order[GROUP_MAX];
        for (int i = 0; i < cnt; i++) order[i] = g0 + i;
        std::stable_sort(order, order + cnt, [&](int x, int y) { return groups[x].M > groups[y].M; });
        int tiles = 0;
        for (int i = 0; i < cnt; i++) {
            const GemmArgs &a = groups[order[i]];
            ga.g[i] = GroupDesc{a.Xq, a.Xs, a.alpha_x, a.X_S, a.Wq, a.Ws, a.alpha_w, a.W_S, a.Y,
                                a.M > 0 ? a.M : 0};
            ga.tile_start[i] = tiles;
            if (ga.g[i].M <= 0) continue;
            tiles += ga.g[i].M <= GROUP_SMALL_M ? (int)((N + GROUP_SMALL_BN - 1) / GROUP_SMALL_BN)
                                                : (int)((ga.g[i].M + BM - 1) / BM) * ga.tiles_n;
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

// SPLIT: the K chunks may be split over sk.nsplit workgroups, each summing a
// contiguous range; the workgroup sums go to the workspace and the last of a
// column group's workgroups to arrive adds them in split order and finishes
// the tiles (the prefill path's fixup).
template <int MB, int CB, int NW, int BB, bool TAIL, bool SPLIT = false>
__device__ __forceinline__ void decode2_body(const GemmArgs &a, int64_t blk, const SplitK &sk = SplitK{})
{
    using C = DecodeCfg<MB, CB, NW, BB>;
    __shared__ f32x4 red[NW][C::RED_TILES][WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int g = lane >> 4, rr = lane & 15;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t rowb = K / 2, rows = K / 16;
    const int64_t n0 = blk * (16 * CB);
    const int nchunk = (int)(K / BK);
    const bool split = SPLIT && sk.nsplit > 1;
    int c_lo = 0, c_hi = nchunk;
    if (split) {
        const int per = (nchunk + sk.nsplit - 1) / sk.nsplit;
        c_lo = sk.split * per;
        c_hi = min(nchunk, c_lo + per);
    }

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

    // scale pairs held as 16-bit values: widened to 32 bits, the compiler
    // masked them where the loop's register copies meet, which waited for
    // the batch just issued
    u32x4 wc0[BB][CB], xc0[BB][MB], wc1[BB][CB], xc1[BB][MB];
    uint16_t ws0[BB][CB], xs0[BB][MB], ws1[BB][CB], xs1[BB][MB];
    auto load = [&](int c, u32x4 (*wc)[CB], uint16_t (*ws)[CB], u32x4 (*xc)[MB], uint16_t (*xs)[MB]) {
#pragma unroll
        for (int b = 0; b < BB; b++) {
            const int ci = min(c + b * NW, c_hi - 1);        // clamped; masked at use
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
    auto compute = [&](int c, u32x4 (*wc)[CB], uint16_t (*ws)[CB], u32x4 (*xc)[MB], uint16_t (*xs)[MB]) {
#pragma unroll
        for (int b = 0; b < BB; b++) {
            const bool ok = c + b * NW < c_hi;
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

    int c = c_lo + wave;
    const bool any = c < c_hi;            // wave-uniform
    if (any) load(c, wc0, ws0, xc0, xs0);
    // W_S fragments (k = 32 or 64) of the tile this wave finishes, issued by
    // every wave alike right behind its first batch: the waits for later
    // batches, younger loads, include them, and by then they have arrived.
    // (Loaded in the epilogue, their HBM latency would add to the call's
    // tail.)  X_S, a few KB that every workgroup reads, comes from L2 in the
    // epilogue.  Only where each wave finishes at most one tile, in one
    // round: two would hold 8 more registers than the widest form can spare.
    constexpr int TPW = (C::T + NW - 1) / NW;
    const int k = a.k;
    // With the K range split, every workgroup of a column group loads them,
    // though only the last to arrive uses them (the splits run side by side
    // on one XCD, so the later loads hit L2) -- where each wave finishes a
    // tile of its own: with fewer tiles than waves, the duplicate loads of
    // all splits cost more than the last workgroup's wait for W_S (k at
    // M = 8: 7.1 against 6.7 us).
    const bool side_pre = TAIL && TPW == 1 && C::RED_TILES == C::T && (k == 32 || k == 64) &&
                          (!split || C::T == NW);
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
    // Two register batches, both in flight from the start: while one batch
    // is decoded and multiplied, the loads of the batch two ahead go into
    // its registers.  The loop runs while four or more batches remain, so
    // each of its loads is real and it has a single exit; the last two or
    // three batches follow it.  (With exits between the batches, or loads
    // that might not be issued, the compiler could not count the younger
    // loads at the top of the loop and waited for all of them, the batch
    // just issued included.)  The scheduling barriers keep the compiler from
    // sinking a batch's loads below the arithmetic before them.
    constexpr int STEP = BB * NW;
    const int nbatch = any ? (c_hi - c + STEP - 1) / STEP : 0;
    if (nbatch == 1) {
        compute(c, wc0, ws0, xc0, xs0);
    } else if (nbatch > 1) {
        load(c + STEP, wc1, ws1, xc1, xs1);
        __builtin_amdgcn_sched_barrier(0);
        int j = 0;
        for (; j + 4 <= nbatch; j += 2) {
            compute(c, wc0, ws0, xc0, xs0);
            load(c + 2 * STEP, wc0, ws0, xc0, xs0);
            __builtin_amdgcn_sched_barrier(0);
            compute(c + STEP, wc1, ws1, xc1, xs1);
            load(c + 3 * STEP, wc1, ws1, xc1, xs1);
            __builtin_amdgcn_sched_barrier(0);
            c += 2 * STEP;
        }
        const int rest = nbatch - j;                           // 2 or 3
        compute(c, wc0, ws0, xc0, xs0);
        if (rest == 3) {
            load(c + 2 * STEP, wc0, ws0, xc0, xs0);
            __builtin_amdgcn_sched_barrier(0);
        }
        compute(c + STEP, wc1, ws1, xc1, xs1);
        if (rest == 3) compute(c + 2 * STEP, wc0, ws0, xc0, xs0);
    }

    // ---- deterministic cross-wave sum through LDS, in rounds of RED_TILES tiles
    const float alpha = (*a.alpha_x) * (*a.alpha_w);
    auto store_tile = [&](int t, const f32x4 &v) {
        const int64_t n = n0 + (t % CB) * 16 + rr;
        if (n < N)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t m = (t / CB) * 16 + g * 4 + q;
                if (m < M) a.Y[m * a.ldy + n] = v[q];
            }
    };
    // tile t's sum v: scale, add the side product, store
    auto finish = [&](int t, f32x4 v) {
        const int i = t / CB, j = t % CB;
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
        store_tile(t, v);
    };
    // split: workgroup sums of tile t from split sp, lane-contiguous 16 bytes
    auto slot = [&](int sp, int t, int h) {
        return reinterpret_cast<uint64_t *>(sk.part) +
               ((((int64_t)sk.wtile * sk.nsplit + sp) * C::T + t) * WAVE + lane) * 2 + h;
    };
#pragma unroll
    for (int t0 = 0; t0 < C::T; t0 += C::RED_TILES) {
        if (t0 > 0) __syncthreads();
#pragma unroll
        for (int t = 0; t < C::RED_TILES; t++)
            if (t0 + t < C::T) red[wave][t][lane] = acc[(t0 + t) / CB][(t0 + t) % CB];
        __syncthreads();
        for (int t = wave; t < C::RED_TILES && t0 + t < C::T; t += NW) {
            f32x4 v = red[0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; w++) v += red[w][t][lane];
            if (split) {
                const f32x2 lo = {v[0], v[1]}, hi = {v[2], v[3]};
                __hip_atomic_store(slot(sk.split, t0 + t, 0), __builtin_bit_cast(uint64_t, lo), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slot(sk.split, t0 + t, 1), __builtin_bit_cast(uint64_t, hi), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            } else {
                finish(t0 + t, v);
            }
        }
    }
    if (SPLIT && split) {
        __shared__ int last_flag;
        wait_vmem();
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(sk.cnt + sk.wtile, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            const bool last = prev == (unsigned)(sk.nsplit - 1);
            if (last) __hip_atomic_store(sk.cnt + sk.wtile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = last;
        }
        __syncthreads();
        if (!last_flag) return;
        // the side fragments (k = 32 or 64: X_S here, W_S since the main
        // loop where each wave finishes one tile), then every split's sums of
        // a tile, are loaded before any is used (loads complete in issue
        // order, so the side loads' latency passes while the sums arrive);
        // the sum runs in split order
        const bool pre = TAIL && (k == 32 || k == 64);
        for (int t = wave; t < C::T; t += NW) {
            bf16x8 sa[2] = {}, sb[2] = {};
            const int64_t n = n0 + (t % CB) * 16 + rr, mrow = (t / CB) * 16 + rr;
            if (pre) {
#pragma unroll
                for (int h = 0; h < 2; h++)
                    if (h * 32 < k) {
                        if (mrow < M)
                            sa[h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(a.X_S + mrow * k + h * 32 + g * 8));
                        if (n < N)
                            sb[h] = side_pre ? tb[h]
                                             : __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(a.W_S + n * k + h * 32 + g * 8));
                    }
            }
            uint64_t p[DECODE_SPLIT_MAX][2];
#pragma unroll
            for (int sp = 0; sp < DECODE_SPLIT_MAX; sp++)
                if (sp < sk.nsplit)
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        p[sp][h] = __hip_atomic_load(slot(sp, t, h), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            f32x4 v;
#pragma unroll
            for (int sp = 0; sp < DECODE_SPLIT_MAX; sp++)
                if (sp < sk.nsplit) {
                    const f32x2 lo = __builtin_bit_cast(f32x2, p[sp][0]), hi = __builtin_bit_cast(f32x2, p[sp][1]);
                    const f32x4 u = {lo.x, lo.y, hi.x, hi.y};
                    v = sp == 0 ? u : v + u;
                }
            if (pre) {
                v *= alpha;
                v = mfma_bf16(sa[0], sb[0], v);
                if (k == 64) v = mfma_bf16(sa[1], sb[1], v);
                store_tile(t, v);
            } else {
                finish(t, v);
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

// K split over workgroups: the splits of a column group are consecutive work
// items, so they usually run on one XCD
template <int MB, int CB, int NW, int BB, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode2s_kernel(GemmArgs a, int nsplit, unsigned *cnt, float *part)
{
    const int item = xcd_order(blockIdx.x, gridDim.x);
    SplitK sk;
    sk.nsplit = nsplit;
    sk.wtile = item / nsplit;
    sk.split = item - (int)sk.wtile * nsplit;
    sk.cnt = cnt;
    sk.part = part;
    decode2_body<MB, CB, NW, BB, TAIL, true>(a, sk.wtile, sk);
}

template <int MB, int CB, int NW, int BB, bool TAIL>
__global__ __launch_bounds__(64 * NW) void decode2s_seg_kernel(SegTable t, int nsplit, unsigned *cnt, float *part)
{
    const int item = xcd_order(blockIdx.x, gridDim.x);
    SplitK sk;
    sk.nsplit = nsplit;
    sk.wtile = item / nsplit;
    sk.split = item - (int)sk.wtile * nsplit;
    sk.cnt = cnt;
    sk.part = part;
    int local;
    const GemmArgs a = seg_args(t, (int)sk.wtile, local);
    decode2_body<MB, CB, NW, BB, TAIL, true>(a, local, sk);
}

template <int MB, int CB, int NW, int BB>
static hipError_t run_decode2s(const GemmArgs &a, const SegSpec *sp, int nsplit, void *ws, hipStream_t s)
{
    unsigned *cnt = static_cast<unsigned *>(ws);
    float *part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + SPLIT_COUNTER_BYTES);
    if (sp) {
        const SegTable t = make_seg_table(a, *sp, 16 * CB);
        const dim3 grid((unsigned)(t.start[t.nseg] * nsplit));
        if (a.k > 0)
            hipLaunchKernelGGL((decode2s_seg_kernel<MB, CB, NW, BB, true>), grid, dim3(64 * NW), 0, s, t, nsplit,
                               cnt, part);
        else
            hipLaunchKernelGGL((decode2s_seg_kernel<MB, CB, NW, BB, false>), grid, dim3(64 * NW), 0, s, t, nsplit,
                               cnt, part);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(((a.N + 16 * CB - 1) / (16 * CB)) * nsplit));
    if (a.k > 0)
        hipLaunchKernelGGL((decode2s_kernel<MB, CB, NW, BB, true>), grid, dim3(64 * NW), 0, s, a, nsplit, cnt, part);
    else
        hipLaunchKernelGGL((decode2s_kernel<MB, CB, NW, BB, false>), grid, dim3(64 * NW), 0, s, a, nsplit, cnt, part);
    return hipGetLastError();
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

// ===========================================================================
// tile columns of the 128-column tiles over the segments of sp (or of a.N)
static int64_t tiles_n128(int64_t N, const GemmSeg *seg, int nseg)
{
    if (!seg) return (N + 127) / 128;
    int64_t t = 0;
    for (int i = 0; i < nseg; i++) t += (seg[i].N + 127) / 128;
    return t;
}

// ===========================================================================
// Configuration choice (plan_gemm) and launch (dispatch_gemm).
// Decode configurations come from measured sweeps on MI355X (Qwen3-8B
// projection shapes, M = 1, 4, 8, 16, 32, 64):
//  - M <= 4 with the FP16 activations fitting 64 KB of LDS: the LDS form,
//    eight waves of four chunks up to K = 4096, sixteen waves beyond;
//  - M <= 16: wide N (>= 8192 columns) 48 columns per workgroup streaming one
//    chunk at a time (N = 12288: 6-9% faster than the single-round form at
//    M = 8-16); K up to 4096 single round, eight waves of four chunks; longer
//    K streaming, 16 columns per workgroup (K = 12288: 25% faster than the
//    single round at M = 4-16, whose sixteen waves hold six chunks each);
//  - M in 17..32: wide N with K <= 4096 the single-round form with 48 columns
//    per workgroup (one workgroup per CU at N = 12288); otherwise streaming
//    over 8 waves;
//  - M in 33..64: streaming, 48 columns per workgroup for wide N.
enum class Kern { P256, P128, XL8_4, XL16_4, XL16_6, XL16_8, D2_1_3, D3_1_1, D2_1_1, D3_2_3_W4,
                  D2_2_1, D2_4_3, D2_4_1, D2_2_3, D2S_1_1, D2S_2_1, D2S_2_4, D2S_4_2 };

struct GemmPlan {
    Path path;
    Kern kern;
    int rows, cols;         // output tile of one workgroup
    PrefillPlan pp;         // tile size (prefill), K split and workspace (both paths)
};

// Decode path, K split over workgroups (decode2s): as many splits as bring
// the column groups to 256 workgroups, at most DECODE_SPLIT_MAX and at most
// one per eight chunks (every wave of a split holds a chunk).  Returns 1 when
// that leaves nothing to split.
static int decode_splits(int64_t colgroups, int nchunk)
{
    const int64_t cap = std::min<int64_t>(DECODE_SPLIT_MAX, nchunk / 8);
    const int64_t s = std::min<int64_t>(cap, 256 / std::max<int64_t>(colgroups, 1));
    return s >= 2 ? (int)s : 1;
}

// column groups of 16*cb columns: over the segments of seg (each rounded up
// alone, as the segment launch counts them), or of N
static int64_t column_groups(int64_t N, const GemmSeg *seg, int nseg, int cb)
{
    const int64_t u = 16 * cb;
    if (!seg) return (N + u - 1) / u;
    int64_t t = 0;
    for (int i = 0; i < nseg; i++) t += (seg[i].N + u - 1) / u;
    return t;
}

// the largest decode split workspace (256 workgroups of 8 tiles) fits the
// allocation-free entry's array
static_assert(SPLIT_COUNTER_BYTES + (size_t)256 * 8 * WAVE * 16 <= SPLICE_NOALLOC_SCRATCH_BYTES, "no-alloc scratch");

static void set_decode_split(GemmPlan &g, Kern kern, int mb, int cb, int64_t N, const GemmSeg *seg, int nseg,
                             int nchunk)
{
    const int64_t cg = column_groups(N, seg, nseg, cb);
    const int ns = decode_splits(cg, nchunk);
    if (ns < 2) return;
    // one arrival counter per column group, in the fixed counter region
    if (cg * 4 > (int64_t)SPLIT_COUNTER_BYTES || mb * cb > 8) return;
    g.kern = kern;
    g.rows = 16 * mb;
    g.cols = 16 * cb;
    g.pp.nsplit = ns;
    g.pp.tiles = cg;
    g.pp.ws = SPLIT_COUNTER_BYTES + (size_t)cg * ns * mb * cb * WAVE * 16;
}

static GemmPlan plan_gemm(Path p, int64_t M, int64_t N, int64_t K, const GemmSeg *seg, int nseg)
{
    GemmPlan g{};
    g.pp = PrefillPlan{false, 1, 0, 0};
    if (K == 0) p = Path::Prefill;      // the decode kernels assume at least one K chunk
    g.path = p;
    if (p == Path::Prefill) {
        // largest tile that still gives every CU a tile, then a K split
        g.pp = plan_prefill(M, N, K, tiles_n128(N, seg, nseg));
        g.kern = g.pp.big ? Kern::P256 : Kern::P128;
        g.rows = g.cols = g.pp.big ? 256 : 128;
        return g;
    }
    const int nchunk = (int)(K / BK);
    const int64_t colblocks = (N + 15) / 16;
    if (M <= 16) {
        g.rows = 16;
        g.cols = 16;
        // 16-byte aligned scale pairs need an even chunk count
        if (M <= 4 && M * K * 2 <= XLDS_MAX && nchunk >= 2 && nchunk % 2 == 0 && nchunk <= 16 * 8) {
            g.kern = nchunk <= 8 * 4 ? Kern::XL8_4 : nchunk <= 16 * 4 ? Kern::XL16_4
                   : nchunk <= 16 * 6 ? Kern::XL16_6 : Kern::XL16_8;
        } else if (colblocks >= 512) {
            g.kern = Kern::D2_1_3;
            g.cols = 48;
        } else {
            g.kern = nchunk <= 32 ? Kern::D3_1_1 : Kern::D2_1_1;
            if (colblocks <= 64) set_decode_split(g, Kern::D2S_1_1, 1, 1, N, seg, nseg, nchunk);
        }
    } else if (M <= 32) {
        g.rows = 32;
        g.cols = 16;
        if (colblocks >= 512 && nchunk <= 4 * 4) {
            g.kern = Kern::D3_2_3_W4;
            g.cols = 48;
        } else if (colblocks >= 512 && nchunk <= 8 * 4) {
            // streaming beat the single round here: gate at M = 32, K = 4096,
            // 15.2 against 16.4 us
            g.kern = Kern::D2_2_3;
            g.cols = 48;
        } else {
            g.kern = Kern::D2_2_1;
            if (colblocks <= 64) set_decode_split(g, Kern::D2S_2_1, 2, 1, N, seg, nseg, nchunk);
            else if (nchunk >= 64) set_decode_split(g, Kern::D2S_2_4, 2, 4, N, seg, nseg, nchunk);
        }
    } else {
        g.rows = 64;
        g.cols = colblocks >= 512 ? 48 : 16;
        g.kern = colblocks >= 512 ? Kern::D2_4_3 : Kern::D2_4_1;
        if (colblocks <= 256) set_decode_split(g, Kern::D2S_4_2, 4, 2, N, seg, nseg, nchunk);
    }
    return g;
}

// launch; sp != nullptr: the column segments of sp, whose widths sum to a.N
static hipError_t dispatch_gemm(Path p, const GemmArgs &a, const SegSpec *sp, void *ws, hipStream_t s)
{
    if (a.M == 0 || a.N == 0) return hipSuccess;
    const GemmPlan g = plan_gemm(p, a.M, a.N, a.K, sp ? sp->seg : nullptr, sp ? sp->nseg : 0);
    const bool t = a.k > 0;
    switch (g.kern) {
    case Kern::P256: return t ? launch_prefill_lds<true>(a, sp, s) : launch_prefill_lds<false>(a, sp, s);
    case Kern::P128: return t ? launch_prefill_lds128<true>(a, sp, g.pp, ws, s) : launch_prefill_lds128<false>(a, sp, g.pp, ws, s);
    case Kern::XL8_4: return run_decode_xlds<8, 4>(a, sp, s);
    case Kern::XL16_4: return run_decode_xlds<16, 4>(a, sp, s);
    case Kern::XL16_6: return run_decode_xlds<16, 6>(a, sp, s);
    case Kern::XL16_8: return run_decode_xlds<16, 8>(a, sp, s);
    case Kern::D2_1_3: return run_decode2<1, 3, 8, 1>(a, sp, s);
    case Kern::D3_1_1: return run_decode3<1, 1, 8, 4>(a, sp, s);
    case Kern::D2_1_1: return run_decode2<1, 1, 8, 1>(a, sp, s);
    case Kern::D3_2_3_W4: return run_decode3<2, 3, 4, 4>(a, sp, s);
    case Kern::D2_2_1: return run_decode2<2, 1, 8, 1>(a, sp, s);
    case Kern::D2_2_3: return run_decode2<2, 3, 8, 1>(a, sp, s);
    case Kern::D2_4_3: return run_decode2<4, 3, 8, 1>(a, sp, s);
    case Kern::D2_4_1: return run_decode2<4, 1, 8, 2>(a, sp, s);
    case Kern::D2S_1_1: return run_decode2s<1, 1, 8, 1>(a, sp, g.pp.nsplit, ws, s);
    case Kern::D2S_2_1: return run_decode2s<2, 1, 8, 1>(a, sp, g.pp.nsplit, ws, s);
    case Kern::D2S_2_4: return run_decode2s<2, 4, 8, 1>(a, sp, g.pp.nsplit, ws, s);
    case Kern::D2S_4_2: return run_decode2s<4, 2, 8, 1>(a, sp, g.pp.nsplit, ws, s);
    }
    return hipErrorInvalidValue;
}

// workspace of a call: the K split's counters and partial sums, or none
size_t gemm_ws_bytes(Path p, int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || (p == Path::Decode && M > SPLICE_DECODE_MAX_M)) return 0;
    return plan_gemm(p, M, N, K, nullptr, 0).pp.ws;
}

size_t gemm_seg_ws_bytes(Path p, int64_t M, int64_t K, const GemmSeg *seg, int nseg)
{
    int64_t N = 0;
    for (int i = 0; i < nseg; i++) N += seg[i].N;
    if (M <= 0 || N <= 0 || K <= 0 || (p == Path::Decode && M > SPLICE_DECODE_MAX_M)) return 0;
    return plan_gemm(p, M, N, K, seg, nseg).pp.ws;
}

void gemm_plan_info(Path p, int64_t M, int64_t N, int64_t K, const GemmSeg *seg, int nseg, int32_t out[5])
{
    const GemmPlan g = plan_gemm(p, M, N, K, seg, nseg);
    out[0] = g.path == Path::Decode ? 1 : 2;
    // every prefill tile size sums K in the same order: one kernel number
    out[1] = g.path == Path::Prefill ? 0 : (int32_t)g.kern;
    out[2] = g.rows;
    out[3] = g.cols;
    out[4] = g.pp.nsplit;
}

hipError_t launch_gemm(Path p, const GemmArgs &a, void *ws, size_t, hipStream_t s)
{
    return dispatch_gemm(p, a, nullptr, ws, s);
}

hipError_t launch_gemm_seg(Path p, const GemmArgs &a, const GemmSeg *seg, int nseg, void *ws, hipStream_t s)
{
    // the configuration is chosen for the combined width, as for one call
    // with N = the sum of the widths
    GemmArgs b = a;
    b.N = 0;
    for (int i = 0; i < nseg; i++) b.N += seg[i].N;
    if (nseg == 0 || b.M == 0 || b.N == 0) return hipSuccess;
    const SegSpec sp{seg, nseg};
    return dispatch_gemm(p, b, &sp, ws, s);
}

}  // namespace splice
