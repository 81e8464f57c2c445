// api.hip -- the C ABI of libsplice.so (declared in include/splice.h):
// host-side argument checks, then launches on the caller's stream.
#include "../../include/splice.h"
#include "kernels.hpp"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include <dlfcn.h>

#include <hip/hip_runtime.h>

using namespace splice;

// ---------------------------------------------------------------------------
// Workspace of splice_gemm_noalloc: a file-scope device array (each GPU holds
// its own copy for the life of the process).  Host code never passes the
// array's name to a kernel -- on the host it only stands for the symbol --
// but the device address hipGetSymbolAddress returns for the current device,
// resolved once per device on the first call there.
static __device__ __align__(256) uint8_t scratch[SPLICE_NOALLOC_SCRATCH_BYTES];

constexpr int SPLIT_COUNTER_WORDS = (int)(SPLIT_COUNTER_BYTES / 4);

__global__ void clear_words_kernel(unsigned *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

namespace {

constexpr int NOALLOC_DEVICES = 64;
std::mutex noalloc_mutex;
void *noalloc_ptr[NOALLOC_DEVICES];

// the device address of `scratch` on the current device; on the first call
// there, its counter words are cleared on `s` ahead of any use
hipError_t noalloc_scratch(hipStream_t s, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= NOALLOC_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(noalloc_mutex);
    if (!noalloc_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(SPLIT_COUNTER_WORDS), 0, s,
                           static_cast<unsigned *>(ptr), SPLIT_COUNTER_WORDS);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        noalloc_ptr[dev] = ptr;
    }
    *out = noalloc_ptr[dev];
    return hipSuccess;
}

constexpr int64_t MAX_K = 65536;

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t hs(splice_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? SPLICE_OK : SPLICE_ERR_HIP; }

// shape rules shared by every entry point
inline int check_k(int64_t K, int32_t k)
{
    if (K < 0 || K % 16 != 0 || k < 0 || k > K) return SPLICE_ERR_INVALID_ARG;
    if (K > MAX_K) return SPLICE_ERR_UNSUPPORTED;
    return SPLICE_OK;
}

int check_gemm(const GemmArgs &a, int path)
{
    if (a.M < 0 || a.N < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(a.K, a.k);
    if (rc) return rc;
    if (path != SPLICE_PATH_AUTO && path != SPLICE_PATH_DECODE && path != SPLICE_PATH_PREFILL)
        return SPLICE_ERR_INVALID_ARG;
    if (path == SPLICE_PATH_DECODE && a.M > SPLICE_DECODE_MAX_M) return SPLICE_ERR_INVALID_ARG;
    if (a.M == 0 || a.N == 0) return SPLICE_OK;
    if (a.ldy < a.N) return SPLICE_ERR_INVALID_ARG;
    if (a.K % 128 != 0) return SPLICE_ERR_UNSUPPORTED;
    if (!a.Y || !a.alpha_x || !a.alpha_w) return SPLICE_ERR_INVALID_ARG;
    if (a.K > 0 && (!a.Xq || !a.Xs || !a.Wq || !a.Ws)) return SPLICE_ERR_INVALID_ARG;
    if (a.k > 0 && (!a.X_S || !a.W_S)) return SPLICE_ERR_INVALID_ARG;
    // the kernels load codes and (in the decode path) scales as 16-byte vectors
    if (!aligned(a.Xq, 16) || !aligned(a.Wq, 16) || !aligned(a.Xs, 16) || !aligned(a.Ws, 16) ||
        !aligned(a.Y, 4))
        return SPLICE_ERR_INVALID_ARG;
    const uintptr_t side_al = (a.k % 8 == 0) ? 16 : 2;
    if (a.k > 0 && (!aligned(a.X_S, side_al) || !aligned(a.W_S, side_al))) return SPLICE_ERR_INVALID_ARG;
    return SPLICE_OK;
}

inline Path choose_path(int64_t M, int path)
{
    if (path == SPLICE_PATH_DECODE) return Path::Decode;
    if (path == SPLICE_PATH_PREFILL) return Path::Prefill;
    return M <= SPLICE_DECODE_MAX_M ? Path::Decode : Path::Prefill;
}

// SPLICE_LOG set to anything but "" or "0" when the library is first used:
// every GEMM call that passes its argument checks writes one line to stderr
// with its shape, the launch its plan chose and the status it returns.
bool log_on()
{
    static const bool on = [] {
        const char *v = std::getenv("SPLICE_LOG");
        return v != nullptr && *v != 0 && std::strcmp(v, "0") != 0;
    }();
    return on;
}

int log_gemm(const char *fn, Path p, int64_t M, int64_t N, int64_t K, int32_t k, const GemmSeg *seg, int nseg,
             int rc)
{
    if (!log_on()) return rc;
    int32_t pl[5] = {0, 0, 0, 0, 0};
    gemm_plan_info(p, M, N, K, seg, nseg, pl);
    std::fprintf(stderr, "[splice] %s M=%lld N=%lld K=%lld k=%d segments=%d path=%s kernel=%d tile=%dx%d "
                 "splits=%d status=%d\n", fn, (long long)M, (long long)N, (long long)K, (int)k, nseg,
                 pl[0] == 1 ? "decode" : "prefill", (int)pl[1], (int)pl[2], (int)pl[3], (int)pl[4], rc);
    return rc;
}

// SPLICE_ROCTX set to anything but "" or "0" when the library is first used:
// every compute entry point runs inside a roctx range named for the call and
// its shape, for profilers that trace markers (rocprofv3 --marker-trace).
// The roctx library is opened at that first use, so the library itself does
// not depend on it; when it cannot be opened the ranges are left out.
struct RoctxApi {
    int (*push)(const char *) = nullptr;
    int (*pop)() = nullptr;
};

const RoctxApi &roctx()
{
    static const RoctxApi api = [] {
        RoctxApi r;
        const char *v = std::getenv("SPLICE_ROCTX");
        if (v == nullptr || *v == 0 || std::strcmp(v, "0") == 0) return r;
        for (const char *name : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so", "libroctx64.so.4",
                                 "libroctx64.so"}) {
            void *h = dlopen(name, RTLD_NOW | RTLD_LOCAL);
            if (!h) continue;
            r.push = reinterpret_cast<int (*)(const char *)>(dlsym(h, "roctxRangePushA"));
            r.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
            if (r.push && r.pop) return r;
            r = RoctxApi{};
        }
        return r;
    }();
    return api;
}

// a roctx range for the lifetime of the object (nothing when SPLICE_ROCTX is off)
class Range {
public:
    explicit Range(const char *fmt, ...) __attribute__((format(printf, 2, 3)))
    {
        const RoctxApi &r = roctx();
        if (!r.push) return;
        char name[160];
        va_list ap;
        va_start(ap, fmt);
        std::vsnprintf(name, sizeof(name), fmt, ap);
        va_end(ap);
        r.push(name);
        on_ = true;
    }
    ~Range()
    {
        if (on_) roctx().pop();
    }
    Range(const Range &) = delete;
    Range &operator=(const Range &) = delete;

private:
    bool on_ = false;
};

int run_gemm(const char *fn, const GemmArgs &a, void *ws, size_t ws_bytes, int path, hipStream_t s)
{
    int rc = check_gemm(a, path);
    if (rc) return rc;
    if (a.M == 0 || a.N == 0) return SPLICE_OK;
    const Path p = choose_path(a.M, path);
    const size_t need = gemm_ws_bytes(p, a.M, a.N, a.K);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 16)))
        return log_gemm(fn, p, a.M, a.N, a.K, a.k, nullptr, 0, SPLICE_ERR_WORKSPACE);
    return log_gemm(fn, p, a.M, a.N, a.K, a.k, nullptr, 0, hip_status(launch_gemm(p, a, ws, ws_bytes, s)));
}

}  // namespace

extern "C" {

const char *splice_status_string(int status)
{
    switch (status) {
    case SPLICE_OK: return "ok";
    case SPLICE_ERR_INVALID_ARG: return "invalid argument";
    case SPLICE_ERR_UNSUPPORTED: return "unsupported shape";
    case SPLICE_ERR_WORKSPACE: return "workspace too small";
    case SPLICE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

size_t splice_select_workspace_size(int64_t) { return 0; }

int splice_select_channels(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int32_t k,
                           int64_t *count, double *mean, double *m2, float *absmax, int32_t *idx,
                           float *alpha_x, void *ws, size_t ws_bytes, splice_stream_t stream)
{
    const Range range("splice_select_channels T=%lld K=%lld k=%d", (long long)T, (long long)K, (int)k);
    (void)ws;
    (void)ws_bytes;
    if (T < 0 || !count || *count < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(K, k);
    if (rc) return rc;
    if (K == 0) {
        *count += T;
        return SPLICE_OK;
    }
    if (!mean || !m2 || !absmax || (k > 0 && !idx) || (T > 0 && !X)) return SPLICE_ERR_INVALID_ARG;
    if (T > 0 && ldx < K) return SPLICE_ERR_INVALID_ARG;
    if (!aligned(X, 2) || !aligned(mean, 8) || !aligned(m2, 8) || !aligned(absmax, 4) ||
        !aligned(idx, 4) || !aligned(alpha_x, 4))
        return SPLICE_ERR_INVALID_ARG;
    hipError_t e = launch_stats(X, T, K, ldx, *count, mean, m2, absmax, hs(stream));
    if (e != hipSuccess) return SPLICE_ERR_HIP;
    e = launch_select(m2, nullptr, *count + T, absmax, K, k, idx, alpha_x, hs(stream));
    if (e != hipSuccess) return SPLICE_ERR_HIP;
    *count += T;
    return SPLICE_OK;
}

int splice_channel_stats(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, int64_t *count,
                         double *mean, double *m2, float *absmax, splice_stream_t stream)
{
    const Range range("splice_channel_stats T=%lld K=%lld", (long long)T, (long long)K);
    if (T < 0 || !count || *count < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(K, 0);
    if (rc) return rc;
    if (K == 0) {
        *count += T;
        return SPLICE_OK;
    }
    if (!mean || !m2 || !absmax || (T > 0 && !X)) return SPLICE_ERR_INVALID_ARG;
    if (T > 0 && ldx < K) return SPLICE_ERR_INVALID_ARG;
    if (!aligned(X, 2) || !aligned(mean, 8) || !aligned(m2, 8) || !aligned(absmax, 4))
        return SPLICE_ERR_INVALID_ARG;
    hipError_t e = launch_stats(X, T, K, ldx, *count, mean, m2, absmax, hs(stream));
    if (e != hipSuccess) return SPLICE_ERR_HIP;
    *count += T;
    return SPLICE_OK;
}

int splice_select_topk(const double *mean, const double *m2, const float *absmax, int64_t count,
                       int64_t K, int32_t k, int criterion, int32_t *idx, float *alpha_x,
                       splice_stream_t stream)
{
    const Range range("splice_select_topk K=%lld k=%d", (long long)K, (int)k);
    if (count < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(K, k);
    if (rc) return rc;
    if (criterion != SPLICE_SELECT_VARIANCE && criterion != SPLICE_SELECT_SECOND_MOMENT)
        return SPLICE_ERR_INVALID_ARG;
    if (K == 0) return SPLICE_OK;
    const bool sm = criterion == SPLICE_SELECT_SECOND_MOMENT;
    if (!m2 || !absmax || (k > 0 && !idx) || (sm && !mean)) return SPLICE_ERR_INVALID_ARG;
    if (!aligned(m2, 8) || !aligned(mean, 8) || !aligned(absmax, 4) || !aligned(idx, 4) ||
        !aligned(alpha_x, 4))
        return SPLICE_ERR_INVALID_ARG;
    return hip_status(launch_select(m2, sm ? mean : nullptr, count, absmax, K, k, idx, alpha_x,
                                    hs(stream)));
}

size_t splice_alpha_workspace_size(void) { return alpha_ws_bytes(); }

int splice_compute_alpha(const uint16_t *A, int64_t R, int64_t K, int64_t lda, const int32_t *idx,
                         int32_t k, float *alpha, void *ws, size_t ws_bytes,
                         splice_stream_t stream)
{
    const Range range("splice_compute_alpha R=%lld K=%lld", (long long)R, (long long)K);
    if (R < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(K, k);
    if (rc) return rc;
    if (!alpha || !aligned(alpha, 4)) return SPLICE_ERR_INVALID_ARG;
    if (R > 0 && K > 0) {
        if (!A || lda < K || (k > 0 && !idx)) return SPLICE_ERR_INVALID_ARG;
        if (!aligned(A, 16) || lda % 8 != 0) return SPLICE_ERR_UNSUPPORTED;
    }
    if (!ws || ws_bytes < alpha_ws_bytes() || !aligned(ws, 4)) return SPLICE_ERR_WORKSPACE;
    return hip_status(launch_alpha(A, R, K, lda, idx, k, alpha, ws, hs(stream)));
}

int splice_quantize_nvfp4(const uint16_t *A, int64_t R, int64_t K, int64_t lda, const int32_t *idx,
                          int32_t k, const float *alpha, uint8_t *codes, uint8_t *scales,
                          uint16_t *side, splice_stream_t stream)
{
    const Range range("splice_quantize_nvfp4 R=%lld K=%lld k=%d", (long long)R, (long long)K, (int)k);
    if (R < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(K, k);
    if (rc) return rc;
    if (R == 0 || K == 0) return SPLICE_OK;
    if (!A || !alpha || !codes || !scales || lda < K || (k > 0 && (!idx || !side)))
        return SPLICE_ERR_INVALID_ARG;
    if (!aligned(A, 16) || lda % 8 != 0) return SPLICE_ERR_UNSUPPORTED;
    if (!aligned(codes, 8) || !aligned(alpha, 4) || (k > 0 && !aligned(side, 2)))
        return SPLICE_ERR_INVALID_ARG;
    return hip_status(launch_quantize(A, R, K, lda, idx, k, alpha, codes, scales, side, hs(stream)));
}

size_t splice_workspace_size(int64_t M, int64_t N, int64_t K, int32_t)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    // enough for whichever path a call takes (the decode path needs none)
    return std::max(gemm_ws_bytes(Path::Decode, M, N, K), gemm_ws_bytes(Path::Prefill, M, N, K));
}

int splice_gemm_plan(int64_t M, int64_t N, int64_t K, int path, int32_t *plan)
{
    if (!plan || M <= 0 || N <= 0 || K < 0 || K % 16 != 0) return SPLICE_ERR_INVALID_ARG;
    if (path != SPLICE_PATH_AUTO && path != SPLICE_PATH_DECODE && path != SPLICE_PATH_PREFILL)
        return SPLICE_ERR_INVALID_ARG;
    if (path == SPLICE_PATH_DECODE && M > SPLICE_DECODE_MAX_M) return SPLICE_ERR_INVALID_ARG;
    gemm_plan_info(choose_path(M, path), M, N, K, nullptr, 0, plan);
    return SPLICE_OK;
}

int splice_multi_plan(int64_t M, int64_t K, const splice_weight_seg *segs, int32_t nseg, int path,
                      int32_t *plan)
{
    if (!plan || !segs || nseg < 1 || nseg > SPLICE_SEG_MAX || M <= 0 || K < 0 || K % 16 != 0)
        return SPLICE_ERR_INVALID_ARG;
    if (path != SPLICE_PATH_AUTO && path != SPLICE_PATH_DECODE && path != SPLICE_PATH_PREFILL)
        return SPLICE_ERR_INVALID_ARG;
    if (path == SPLICE_PATH_DECODE && M > SPLICE_DECODE_MAX_M) return SPLICE_ERR_INVALID_ARG;
    GemmSeg seg[SEG_MAX];
    int64_t N = 0;
    for (int32_t i = 0; i < nseg; i++) {
        if (segs[i].N < 0) return SPLICE_ERR_INVALID_ARG;
        seg[i] = GemmSeg{nullptr, nullptr, nullptr, nullptr, nullptr, 0, segs[i].N};
        N += segs[i].N;
    }
    if (N == 0) return SPLICE_ERR_INVALID_ARG;
    gemm_plan_info(choose_path(M, path), M, N, K, seg, nseg, plan);
    return SPLICE_OK;
}

size_t splice_multi_workspace_size(int64_t M, int64_t K, int32_t, const splice_weight_seg *segs,
                                   int32_t nseg)
{
    if (M <= 0 || K <= 0 || !segs || nseg < 1 || nseg > SPLICE_SEG_MAX) return 0;
    GemmSeg seg[SEG_MAX];
    for (int32_t i = 0; i < nseg; i++)
        seg[i] = GemmSeg{nullptr, nullptr, nullptr, nullptr, nullptr, 0, segs[i].N > 0 ? segs[i].N : 0};
    return std::max(gemm_seg_ws_bytes(Path::Decode, M, K, seg, nseg),
                    gemm_seg_ws_bytes(Path::Prefill, M, K, seg, nseg));
}

int splice_gemm(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint16_t *X_S,
                const uint8_t *Wq, const uint8_t *Ws, const float *alpha_w, const uint16_t *W_S,
                int64_t M, int64_t N, int64_t K, int32_t k, float *Y, int64_t ldy, void *ws,
                size_t ws_bytes, int path, splice_stream_t stream)
{
    const Range range("splice_gemm M=%lld N=%lld K=%lld k=%d", (long long)M, (long long)N, (long long)K, (int)k);
    GemmArgs a{Xq, Xs, alpha_x, X_S, Wq, Ws, alpha_w, W_S, M, N, K, k, Y, ldy};
    return run_gemm("splice_gemm", a, ws, ws_bytes, path, hs(stream));
}

int splice_gemm_noalloc(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint16_t *X_S,
                        const uint8_t *Wq, const uint8_t *Ws, const float *alpha_w, const uint16_t *W_S,
                        int64_t M, int64_t N, int64_t K, int32_t k, float *Y, int64_t ldy, int path,
                        splice_stream_t stream)
{
    const Range range("splice_gemm_noalloc M=%lld N=%lld K=%lld k=%d", (long long)M, (long long)N, (long long)K, (int)k);
    GemmArgs a{Xq, Xs, alpha_x, X_S, Wq, Ws, alpha_w, W_S, M, N, K, k, Y, ldy};
    int rc = check_gemm(a, path);
    if (rc) return rc;
    if (a.M == 0 || a.N == 0) return SPLICE_OK;
    const Path p = choose_path(a.M, path);
    const size_t need = gemm_ws_bytes(p, a.M, a.N, a.K);
    if (need > SPLICE_NOALLOC_SCRATCH_BYTES)
        return log_gemm("splice_gemm_noalloc", p, M, N, K, k, nullptr, 0, SPLICE_ERR_WORKSPACE);
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = noalloc_scratch(hs(stream), &ws);
        if (e != hipSuccess) return log_gemm("splice_gemm_noalloc", p, M, N, K, k, nullptr, 0, SPLICE_ERR_HIP);
    }
    return log_gemm("splice_gemm_noalloc", p, M, N, K, k, nullptr, 0,
                    hip_status(launch_gemm(p, a, ws, need, hs(stream))));
}

int nvfp4_gemm(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint8_t *Wq,
               const uint8_t *Ws, const float *alpha_w, int64_t M, int64_t N, int64_t K, float *Y,
               int64_t ldy, void *ws, size_t ws_bytes, int path, splice_stream_t stream)
{
    const Range range("nvfp4_gemm M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
    GemmArgs a{Xq, Xs, alpha_x, nullptr, Wq, Ws, alpha_w, nullptr, M, N, K, 0, Y, ldy};
    return run_gemm("nvfp4_gemm", a, ws, ws_bytes, path, hs(stream));
}

int splice_gemm_multi(const uint8_t *Xq, const uint8_t *Xs, const float *alpha_x, const uint16_t *X_S,
                      int64_t M, int64_t K, int32_t k, const splice_weight_seg *segs, int32_t nseg,
                      void *ws, size_t ws_bytes, int path, splice_stream_t stream)
{
    const Range range("splice_gemm_multi M=%lld K=%lld k=%d segments=%d", (long long)M, (long long)K, (int)k, (int)nseg);
    static_assert(SPLICE_SEG_MAX == SEG_MAX, "segment limit");
    if (nseg < 1 || nseg > SPLICE_SEG_MAX || !segs) return SPLICE_ERR_INVALID_ARG;
    GemmSeg seg[SEG_MAX];
    int64_t total = 0;
    for (int32_t i = 0; i < nseg; i++) {
        const splice_weight_seg &w = segs[i];
        GemmArgs a{Xq, Xs, alpha_x, X_S, w.Wq, w.Ws, w.alpha_w, w.W_S, M, w.N, K, k, w.Y, w.ldy};
        int rc = check_gemm(a, path);
        if (rc) return rc;
        seg[i] = GemmSeg{w.Wq, w.Ws, w.alpha_w, w.W_S, w.Y, w.ldy, w.N};
        total += w.N;
    }
    if (total > (int64_t)1 << 30) return SPLICE_ERR_UNSUPPORTED;   // launch units fit an int
    if (M == 0 || total == 0) return SPLICE_OK;
    const Path p = choose_path(M, path);
    const size_t need = gemm_seg_ws_bytes(p, M, K, seg, nseg);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 16)))
        return log_gemm("splice_gemm_multi", p, M, total, K, k, seg, nseg, SPLICE_ERR_WORKSPACE);
    GemmArgs base{Xq, Xs, alpha_x, X_S, nullptr, nullptr, nullptr, nullptr, M, total, K, k, nullptr, 0};
    return log_gemm("splice_gemm_multi", p, M, total, K, k, seg, nseg,
                    hip_status(launch_gemm_seg(p, base, seg, nseg, ws, hs(stream))));
}

int splice_gemm_decode_fused(const uint16_t *X, int64_t ldx, const int32_t *idx,
                             const float *alpha_x, const uint8_t *Wq, const uint8_t *Ws,
                             const float *alpha_w, const uint16_t *W_S, int64_t M, int64_t N,
                             int64_t K, int32_t k, float *Y, int64_t ldy, splice_stream_t stream)
{
    const Range range("splice_gemm_decode_fused M=%lld N=%lld K=%lld k=%d", (long long)M, (long long)N, (long long)K, (int)k);
    if (M < 0 || N < 0) return SPLICE_ERR_INVALID_ARG;
    int rc = check_k(K, k);
    if (rc) return rc;
    if (M > SPLICE_FUSED_MAX_M) return SPLICE_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return SPLICE_OK;
    if (!Y || !alpha_x || !alpha_w || ldy < N) return SPLICE_ERR_INVALID_ARG;
    if (!aligned(Y, 4) || !aligned(alpha_x, 4) || !aligned(alpha_w, 4)) return SPLICE_ERR_INVALID_ARG;
    if (K > 0) {
        if (!X || !Wq || !Ws || ldx < K || (k > 0 && (!idx || !W_S))) return SPLICE_ERR_INVALID_ARG;
        if (!fused_decode_ok(M, K)) return SPLICE_ERR_UNSUPPORTED;
        if (!aligned(X, 16) || ldx % 8 != 0) return SPLICE_ERR_UNSUPPORTED;
        if (!aligned(Wq, 16) || !aligned(Ws, 16) || (k > 0 && !aligned(idx, 4)))
            return SPLICE_ERR_INVALID_ARG;
        if (k > 0 && !aligned(W_S, (k % 8 == 0) ? 16 : 2)) return SPLICE_ERR_INVALID_ARG;
    }
    GemmArgs a{nullptr, nullptr, alpha_x, nullptr, Wq, Ws, alpha_w, W_S, M, N, K, k, Y, ldy,
               X, ldx, idx};
    return hip_status(launch_gemm_fused(a, hs(stream)));
}

int splice_gemm_decode_fused_multi(const uint16_t *X, int64_t ldx, const int32_t *idx,
                                   const float *alpha_x, int64_t M, int64_t K, int32_t k,
                                   const splice_weight_seg *segs, int32_t nseg, splice_stream_t stream)
{
    const Range range("splice_gemm_decode_fused_multi M=%lld K=%lld k=%d segments=%d", (long long)M, (long long)K, (int)k, (int)nseg);
    if (nseg < 1 || nseg > SPLICE_SEG_MAX || !segs) return SPLICE_ERR_INVALID_ARG;
    GemmSeg seg[SEG_MAX];
    int64_t total = 0;
    for (int32_t i = 0; i < nseg; i++) {
        const splice_weight_seg &w = segs[i];
        // each segment as its own fused call would be checked
        if (M < 0 || w.N < 0) return SPLICE_ERR_INVALID_ARG;
        int rc = check_k(K, k);
        if (rc) return rc;
        if (M > SPLICE_FUSED_MAX_M) return SPLICE_ERR_UNSUPPORTED;
        if (M > 0 && w.N > 0) {
            if (!w.Y || !alpha_x || !w.alpha_w || w.ldy < w.N) return SPLICE_ERR_INVALID_ARG;
            if (!aligned(w.Y, 4) || !aligned(alpha_x, 4) || !aligned(w.alpha_w, 4))
                return SPLICE_ERR_INVALID_ARG;
            if (K > 0) {
                if (!X || !w.Wq || !w.Ws || ldx < K || (k > 0 && (!idx || !w.W_S)))
                    return SPLICE_ERR_INVALID_ARG;
                if (!fused_decode_ok(M, K)) return SPLICE_ERR_UNSUPPORTED;
                if (!aligned(X, 16) || ldx % 8 != 0) return SPLICE_ERR_UNSUPPORTED;
                if (!aligned(w.Wq, 16) || !aligned(w.Ws, 16) || (k > 0 && !aligned(idx, 4)))
                    return SPLICE_ERR_INVALID_ARG;
                if (k > 0 && !aligned(w.W_S, (k % 8 == 0) ? 16 : 2)) return SPLICE_ERR_INVALID_ARG;
            }
        }
        seg[i] = GemmSeg{w.Wq, w.Ws, w.alpha_w, w.W_S, w.Y, w.ldy, w.N};
        total += w.N;
    }
    if (total > (int64_t)1 << 30) return SPLICE_ERR_UNSUPPORTED;
    if (M == 0 || total == 0) return SPLICE_OK;
    GemmArgs base{nullptr, nullptr, alpha_x, nullptr, nullptr, nullptr, nullptr, nullptr, M, total, K, k,
                  nullptr, 0, X, ldx, idx};
    return hip_status(launch_gemm_fused_seg(base, seg, nseg, hs(stream)));
}

int splice_tim_filter(const float *logp, int64_t B, int64_t ldl, const int32_t *len, float log_tau,
                      int64_t k1_num, int64_t k1_den, int64_t k2, uint8_t *keep, int32_t *g1,
                      int32_t *g2, float *adv, int64_t adv_cols, int64_t lda,
                      splice_stream_t stream)
{
    const Range range("splice_tim_filter B=%lld", (long long)B);
    constexpr int64_t I31 = 2147483647;
    if (B < 0 || ldl < 0 || k1_num < 0 || k1_den <= 0 || k2 < 0 || adv_cols < 0)
        return SPLICE_ERR_INVALID_ARG;
    if (B > I31 || ldl > I31 || k1_num > I31 || k1_den > I31) return SPLICE_ERR_UNSUPPORTED;
    if (B == 0) return SPLICE_OK;
    if (!len || (ldl > 0 && !logp) || (adv_cols > 0 && (!adv || lda < adv_cols)))
        return SPLICE_ERR_INVALID_ARG;
    if (!aligned(logp, 4) || !aligned(len, 4) || !aligned(g1, 4) || !aligned(g2, 4) ||
        !aligned(adv, 4))
        return SPLICE_ERR_INVALID_ARG;
    TimArgs a{logp, B, ldl, len, log_tau, k1_num, k1_den, k2, keep, g1, g2,
              adv_cols > 0 ? adv : nullptr, adv_cols, lda};
    return hip_status(launch_tim_filter(a, hs(stream)));
}

int splice_probe_mfma_f16(int64_t iters, int64_t workgroups, float *sink, splice_stream_t stream)
{
    if (iters < 0 || workgroups <= 0 || workgroups > 65536 || !sink || !aligned(sink, 4))
        return SPLICE_ERR_INVALID_ARG;
    return hip_status(launch_mfma_rate(iters, workgroups, sink, hs(stream)));
}

int splice_probe_stream_read(const void *src, int64_t bytes, int64_t workgroups, uint32_t *sink,
                             splice_stream_t stream)
{
    if (bytes < 0 || bytes % 16 != 0 || workgroups <= 0 || workgroups > 65536 || !sink ||
        !aligned(sink, 4) || (bytes > 0 && (!src || !aligned(src, 16))))
        return SPLICE_ERR_INVALID_ARG;
    return hip_status(launch_stream_read(src, bytes, workgroups, sink, hs(stream)));
}

size_t splice_grouped_workspace_size(const splice_group *, int32_t, int64_t, int64_t, int32_t)
{
    return 0;
}

int splice_gemm_grouped(const splice_group *groups, int32_t G, int64_t N, int64_t K, int32_t k,
                        void *, size_t, splice_stream_t stream)
{
    const Range range("splice_gemm_grouped groups=%d N=%lld K=%lld k=%d", (int)G, (long long)N, (long long)K, (int)k);
    if (G < 0 || (G > 0 && !groups)) return SPLICE_ERR_INVALID_ARG;
    std::vector<GemmArgs> args;
    args.reserve(G);
    for (int32_t i = 0; i < G; i++) {
        const splice_group &g = groups[i];
        GemmArgs a{g.Xq, g.Xs, g.alpha_x, g.X_S, g.Wq, g.Ws, g.alpha_w, g.W_S, g.M, N, K, k, g.Y, N};
        int rc = check_gemm(a, SPLICE_PATH_PREFILL);
        if (rc) return rc;
        args.push_back(a);
    }
    if (G == 0 || N == 0) return SPLICE_OK;
    return hip_status(launch_gemm_grouped(args.data(), G, hs(stream)));
}

}  // extern "C"
