"""Plans of the GEMM calls on the CPU (splice_gemm_plan / splice_multi_plan):
which path, tile and K split a call of a given shape takes.  Nothing runs on a
GPU."""
import pytest

from fp4_gemm_sparse_amd import splice as S


def test_decode_and_prefill_paths():
    assert S.gemm_plan(1, 4096, 4096)[0] == 1 and S.gemm_plan(64, 4096, 4096)[0] == 1
    assert S.gemm_plan(65, 4096, 4096)[0] == 2
    assert S.gemm_plan(8, 4096, 4096, S.PATH_PREFILL)[0] == 2
    # the timed prefill step: 256 x 256 tiles, no K split
    for N, K in ((4096, 4096), (12288, 4096), (4096, 12288)):
        path, kern, rows, cols, ns = S.gemm_plan(8192, N, K)
        assert (path, rows, cols, ns) == (2, 256, 256, 1)


@pytest.mark.parametrize("M", [65, 128, 256, 512])
@pytest.mark.parametrize("N", [1024, 4096])
def test_small_grids_split_k(M, N):
    """At up to 128 tiles of 128 x 128 the K sum is split as many ways as keep
    the workgroups within 256 and each split at least eight 64-channel steps;
    the workspace holds one partial tile per split."""
    K = 4096
    path, kern, rows, cols, ns = S.gemm_plan(M, N, K)
    tiles = -(-M // 128) * -(-N // 128)
    assert (path, rows, cols) == (2, 128, 128)
    assert ns == (max(1, min(256 // tiles, K // 64 // 8)) if tiles <= 128 else 1)
    assert tiles * ns <= 256
    if ns > 1:
        assert S.workspace_size(M, N, K) >= tiles * ns * 128 * 128 * 4


def test_mid_range_plans():
    """q, k and down at 512 rows split (128, 32 and 128 tiles); gate at 256
    rows (192 tiles) and q at 2048 rows (512 tiles) fill the GPU unsplit."""
    assert S.gemm_plan(512, 4096, 4096)[4] == 2
    assert S.gemm_plan(512, 1024, 4096)[4] == 8
    assert S.gemm_plan(512, 4096, 12288)[4] == 2
    assert S.gemm_plan(256, 12288, 4096)[4] == 1
    assert S.gemm_plan(2048, 4096, 4096)[1:] == (0, 128, 128, 1)


def test_decode_split_plans():
    """Decode path: the K range is split where the column groups alone leave
    CUs idle -- narrow N at 5..64 rows, deep K at 17..32 rows, N <= 4096 at
    33..64 rows -- as many ways as bring the grid to 256 workgroups, at most
    8 and at most one per eight chunks."""
    q, k, gate, down = (4096, 4096), (1024, 4096), (12288, 4096), (4096, 12288)
    expect = {  # M: {shape: (rows, cols, splits)}
        4: {q: (16, 16, 1), k: (16, 16, 1), gate: (16, 16, 1), down: (16, 16, 1)},
        8: {q: (16, 16, 1), k: (16, 16, 4), gate: (16, 48, 1), down: (16, 16, 1)},
        16: {q: (16, 16, 1), k: (16, 16, 4), gate: (16, 48, 1), down: (16, 16, 1)},
        32: {q: (32, 16, 1), k: (32, 16, 4), gate: (32, 48, 1), down: (32, 64, 4)},
        64: {q: (64, 32, 2), k: (64, 32, 4), gate: (64, 48, 1), down: (64, 32, 2)},
    }
    for M, shapes in expect.items():
        for (N, K), want in shapes.items():
            path, kern, rows, cols, ns = S.gemm_plan(M, N, K, S.PATH_DECODE)
            assert (path, rows, cols, ns) == (1,) + want, (M, N, K)
            if ns > 1:
                cg = -(-N // cols)
                assert S.workspace_size(M, N, K) >= 1024 + cg * ns * rows * cols * 4


def test_decode_split_counts_stay_in_bounds():
    for M in (5, 8, 16, 17, 24, 32, 33, 48, 64):
        for N in (16, 64, 500, 1000, 1024, 2100, 4096, 4100, 12288):
            for K in (128, 1024, 2048, 4096, 5248, 8192, 12288, 17408, 65536):
                ns = S.gemm_plan(M, N, K, S.PATH_DECODE)[4]
                cols = S.gemm_plan(M, N, K, S.PATH_DECODE)[3]
                nchunk = K // 128
                assert 1 <= ns <= 8 and ns <= max(1, nchunk // 8)
                cg = -(-N // cols)
                assert ns == 1 or cg * ns <= 256
                per = -(-nchunk // ns)
                assert (ns - 1) * per < nchunk, (M, N, K, ns)


def test_big_tile_when_small_tiles_need_two_rounds():
    """Below 240 tiles of 256 x 256 the big tile still runs when the 128 x 128
    grid needs more than one round (more than 512 tiles): gate at M = 768 and
    1024, a 1536-column gate shard at M = 8192, q at M = 3072; at 512 small
    tiles or fewer the small tile stays (q at M = 2048, gate at M = 512)."""
    for M, N in ((768, 12288), (1024, 12288), (8192, 1536), (3072, 4096)):
        assert S.gemm_plan(M, N, 4096)[2:] == (256, 256, 1), (M, N)
    for M, N in ((2048, 4096), (512, 12288), (8192, 512), (1024, 4096)):
        assert S.gemm_plan(M, N, 4096)[2] == 128, (M, N)


def test_split_ranges_are_never_empty():
    for K in (512, 640, 1152, 4096, 12288, 17408):
        for M, N in ((65, 64), (128, 1024), (200, 300)):
            ns = S.gemm_plan(M, N, K)[4]
            steps = K // 64
            per = -(-steps // ns)
            assert (ns - 1) * per < steps, (M, N, K, ns)


def test_multi_plan_counts_tiles_per_segment():
    # q|k|v at 512 rows: 4 x 48 tiles together, not split; k alone: 32 tiles, eight K ranges
    p_multi = S.multi_plan(512, 4096, [4096, 1024, 1024])
    assert p_multi[4] == 1 and S.gemm_plan(512, 1024, 4096)[4] == 8
    # decode: the combined width chooses the column grouping
    assert S.multi_plan(8, 4096, [12288, 12288])[3] == 48


def test_plan_argument_errors():
    L = S.lib()
    import ctypes
    out = (ctypes.c_int32 * 5)()
    assert L.splice_gemm_plan(0, 16, 128, 0, out) == S.ERR_INVALID_ARG
    assert L.splice_gemm_plan(4, 16, 100, 0, out) == S.ERR_INVALID_ARG
    assert L.splice_gemm_plan(65, 16, 128, S.PATH_DECODE, out) == S.ERR_INVALID_ARG
    assert L.splice_gemm_plan(4, 16, 128, 9, out) == S.ERR_INVALID_ARG
    assert L.splice_gemm_plan(4, 16, 128, 0, None) == S.ERR_INVALID_ARG
