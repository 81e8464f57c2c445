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
