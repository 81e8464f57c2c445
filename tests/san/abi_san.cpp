// Drives the host side of libsplice's C ABI -- argument checks, plans,
// workspace sizes, segment and group tables -- for a build whose host code
// carries AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py).  Nothing here reaches a GPU: every call either
// is a pure host query or is rejected before anything is enqueued.  Exit
// status 0: every call returned what the header promises and the sanitizers
// found nothing.
#include "../../include/splice.h"

#include <cstdint>
#include <cstdio>
#include <vector>

static int failures = 0;
#define CHECK(c)                                                                \
    do {                                                                        \
        if (!(c)) {                                                             \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            failures++;                                                         \
        }                                                                       \
    } while (0)

// a 16-byte aligned non-null address that is never dereferenced
static void *const F = reinterpret_cast<void *>(uintptr_t(0x100000));
template <class T> static T *f(uintptr_t off = 0) { return reinterpret_cast<T *>(uintptr_t(F) + off); }

static int gemm(int64_t M, int64_t N, int64_t K, int32_t k, int path = SPLICE_PATH_AUTO, int64_t ldy = -1,
                void *ws = nullptr, size_t wsb = 0, uintptr_t xq_off = 0)
{
    return splice_gemm(f<uint8_t>(xq_off), f<uint8_t>(), f<float>(), f<uint16_t>(), f<uint8_t>(), f<uint8_t>(),
                       f<float>(), f<uint16_t>(), M, N, K, k, f<float>(), ldy < 0 ? N : ldy, ws, wsb, path,
                       nullptr);
}

int main()
{
    for (int c = -6; c <= 2; c++) CHECK(splice_status_string(c) != nullptr);

    // GEMM argument errors, all caught on the host
    CHECK(gemm(8, 64, 100, 8) == SPLICE_ERR_INVALID_ARG);          // K % 16
    CHECK(gemm(8, 64, 256, 257) == SPLICE_ERR_INVALID_ARG);        // k > K
    CHECK(gemm(-1, 64, 256, 8) == SPLICE_ERR_INVALID_ARG);
    CHECK(gemm(8, 64, 144, 8) == SPLICE_ERR_UNSUPPORTED);          // K % 128
    CHECK(gemm(8, 64, 131072, 8) == SPLICE_ERR_UNSUPPORTED);
    CHECK(gemm(65, 64, 256, 8, SPLICE_PATH_DECODE) == SPLICE_ERR_INVALID_ARG);
    CHECK(gemm(8, 64, 256, 8, 7) == SPLICE_ERR_INVALID_ARG);
    CHECK(gemm(8, 64, 256, 8, SPLICE_PATH_AUTO, 10) == SPLICE_ERR_INVALID_ARG);   // ldy < N
    CHECK(gemm(8, 64, 256, 8, SPLICE_PATH_AUTO, -1, nullptr, 0, 4) == SPLICE_ERR_INVALID_ARG);
    CHECK(gemm(0, 64, 256, 8) == SPLICE_OK);                       // no-op
    CHECK(gemm(128, 1024, 4096, 64) == SPLICE_ERR_WORKSPACE);      // split prefill, no workspace
    CHECK(gemm(64, 1024, 4096, 64, SPLICE_PATH_DECODE) == SPLICE_ERR_WORKSPACE);   // split decode

    // plans and workspace sizes over a grid of shapes, both paths
    const int64_t Ms[] = {1, 3, 4, 5, 8, 16, 17, 32, 33, 64, 65, 128, 300, 2048, 8192, 32768};
    const int64_t Ns[] = {1, 16, 100, 1000, 1024, 4096, 12288, 24576};
    const int64_t Ks[] = {0, 128, 1024, 4096, 5248, 12288, 17408, 65536};
    int32_t plan[5];
    for (int64_t M : Ms)
        for (int64_t N : Ns)
            for (int64_t K : Ks) {
                CHECK(splice_gemm_plan(M, N, K, SPLICE_PATH_AUTO, plan) == SPLICE_OK);
                CHECK(plan[0] == (M <= 64 && K > 0 ? 1 : 2) && plan[4] >= 1);
                CHECK(splice_gemm_plan(M, N, K, SPLICE_PATH_PREFILL, plan) == SPLICE_OK);
                if (M <= 64) CHECK(splice_gemm_plan(M, N, K, SPLICE_PATH_DECODE, plan) == SPLICE_OK);
                CHECK(splice_workspace_size(M, N, K, 64) <= SPLICE_NOALLOC_SCRATCH_BYTES);
            }
    CHECK(splice_gemm_plan(8, 64, 100, SPLICE_PATH_AUTO, plan) == SPLICE_ERR_INVALID_ARG);
    CHECK(splice_gemm_plan(8, 64, 128, SPLICE_PATH_AUTO, nullptr) == SPLICE_ERR_INVALID_ARG);
    CHECK(splice_gemm_plan(65, 64, 128, SPLICE_PATH_DECODE, plan) == SPLICE_ERR_INVALID_ARG);

    // segment tables: ragged widths, an empty segment, the most segments
    std::vector<splice_weight_seg> segs(SPLICE_SEG_MAX + 1);
    for (int i = 0; i <= SPLICE_SEG_MAX; i++)
        segs[i] = splice_weight_seg{f<uint8_t>(), f<uint8_t>(), f<float>(), f<uint16_t>(), 17 + 300 * (i % 3),
                                    f<float>(), 17 + 300 * (i % 3)};
    segs[2].N = 0;
    for (int64_t M : Ms)
        for (int n = 1; n <= SPLICE_SEG_MAX; n++) {
            CHECK(splice_multi_plan(M, 4096, segs.data(), n, SPLICE_PATH_AUTO, plan) == SPLICE_OK);
            CHECK(splice_multi_workspace_size(M, 4096, 64, segs.data(), n) <= SPLICE_NOALLOC_SCRATCH_BYTES);
        }
    CHECK(splice_multi_plan(8, 4096, segs.data(), SPLICE_SEG_MAX + 1, SPLICE_PATH_AUTO, plan) ==
          SPLICE_ERR_INVALID_ARG);
    CHECK(splice_gemm_multi(f<uint8_t>(), f<uint8_t>(), f<float>(), f<uint16_t>(), 8, 4096, 64, segs.data(),
                            SPLICE_SEG_MAX + 1, nullptr, 0, SPLICE_PATH_AUTO, nullptr) == SPLICE_ERR_INVALID_ARG);
    CHECK(splice_gemm_multi(f<uint8_t>(), f<uint8_t>(), f<float>(), f<uint16_t>(), 8, 100, 64, segs.data(), 3,
                            nullptr, 0, SPLICE_PATH_AUTO, nullptr) == SPLICE_ERR_INVALID_ARG);

    // groups: a table of more groups than one launch takes, bad shapes
    std::vector<splice_group> groups(70);
    for (int i = 0; i < 70; i++)
        groups[i] = splice_group{f<uint8_t>(), f<uint8_t>(), f<float>(), f<uint16_t>(), f<uint8_t>(),
                                 f<uint8_t>(), f<float>(), f<uint16_t>(), (int64_t)(i * 37 % 300), f<float>()};
    CHECK(splice_grouped_workspace_size(groups.data(), 70, 2048, 4096, 64) == 0);
    CHECK(splice_gemm_grouped(groups.data(), 70, 2048, 100, 64, nullptr, 0, nullptr) == SPLICE_ERR_INVALID_ARG);
    groups[5].M = -1;
    CHECK(splice_gemm_grouped(groups.data(), 70, 2048, 4096, 64, nullptr, 0, nullptr) == SPLICE_ERR_INVALID_ARG);

    // preparation and filter entry points: argument errors
    CHECK(splice_quantize_nvfp4(f<uint16_t>(), 4, 100, 100, f<int32_t>(), 0, f<float>(), f<uint8_t>(),
                                f<uint8_t>(), nullptr, nullptr) == SPLICE_ERR_INVALID_ARG);
    CHECK(splice_quantize_nvfp4(f<uint16_t>(), 4, 64, 32, f<int32_t>(), 0, f<float>(), f<uint8_t>(),
                                f<uint8_t>(), nullptr, nullptr) == SPLICE_ERR_INVALID_ARG);   // lda < K
    CHECK(splice_compute_alpha(f<uint16_t>(), 4, 64, 64, f<int32_t>(), 65, f<float>(), F, 1 << 20, nullptr) ==
          SPLICE_ERR_INVALID_ARG);
    int64_t count = 0;
    CHECK(splice_select_channels(f<uint16_t>(), 4, 64, 64, 65, &count, f<double>(), f<double>(), f<float>(),
                                 f<int32_t>(), f<float>(), F, splice_select_workspace_size(64), nullptr) ==
          SPLICE_ERR_INVALID_ARG);
    CHECK(splice_select_topk(f<double>(), f<double>(), f<float>(), 0, 64, 65, SPLICE_SELECT_VARIANCE,
                             f<int32_t>(), nullptr, nullptr) == SPLICE_ERR_INVALID_ARG);
    CHECK(splice_select_topk(f<double>(), f<double>(), f<float>(), 0, 64, 4, 9, f<int32_t>(), nullptr,
                             nullptr) == SPLICE_ERR_INVALID_ARG);
    CHECK(splice_gemm_decode_fused(f<uint16_t>(), 4096, f<int32_t>(), f<float>(), f<uint8_t>(), f<uint8_t>(),
                                   f<float>(), f<uint16_t>(), 5, 1024, 4096, 64, f<float>(), 1024, nullptr) ==
          SPLICE_ERR_UNSUPPORTED);
    CHECK(splice_tim_filter(f<float>(), 4, 10, f<int32_t>(), -9.2f, 1, 0, 5, nullptr, nullptr, nullptr,
                            nullptr, 0, 0, nullptr) == SPLICE_ERR_INVALID_ARG);   // k1_den = 0
    CHECK(splice_gemm_noalloc(f<uint8_t>(), f<uint8_t>(), f<float>(), f<uint16_t>(), f<uint8_t>(),
                              f<uint8_t>(), f<float>(), f<uint16_t>(), 8, 64, 100, 8, f<float>(), 64,
                              SPLICE_PATH_AUTO, nullptr) == SPLICE_ERR_INVALID_ARG);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("ABI sanitizer run: ok\n");
    return 0;
}
