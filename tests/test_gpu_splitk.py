"""GPU parity where the K sum is split over workgroups, through the C ABI: the
prefill path (M from 65 to a few hundred rows: the 128 x 128 tile grid alone
would leave CUs idle) and the decode path (narrow N or deep K at 5..64 rows:
the column groups alone would leave CUs idle).

Each split's partial tile goes to the workspace and the workgroup completing a
tile's arrival count sums the partials in split order, so the result must not
depend on which workgroup arrives last: repeated calls give the same bits, a
call after calls of other shapes on the same workspace gives the same bits,
and replays of a captured graph give the eager call's bits.  Against the
oracle: the tolerance in gpu_util.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth
from gpu_util import assert_gemm_close, dev, host, scalar

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def gpu_packs(X_warm, X, W, k):
    idx, ax, _ = S.select_channels(dev(X_warm), k)
    Wd = dev(W)
    aw = S.compute_alpha(Wd, idx)
    return idx, ax, aw, S.quantize_nvfp4(dev(X), idx, ax), S.quantize_nvfp4(Wd, idx, aw)


@pytest.mark.parametrize("M", [65, 128, 256, 512, 2048])
@pytest.mark.parametrize("name", ["q", "k", "down"])
def test_split_prefill_full_size_sampled(name, M):
    """Qwen3-8B projections at M rows (prefill workload distributions) from
    just above the decode path to 2048 rows: the plan splits K where the
    grid has at most 128 tiles of 128 x 128 (every case here but q and down
    at 2048 rows), and 160 sampled output columns meet the oracle's own
    calibration, packs and product."""
    p = synth.projection(synth.CFG_PREFILL, name, M)
    K, N = p["K"], p["N"]
    tiles = -(-M // 128) * -(-N // 128)
    assert (S.gemm_plan(M, N, K)[4] > 1) == (tiles <= 128)
    cols = np.sort(np.random.default_rng(M + N).choice(N, size=160, replace=False))
    idx_o, ax_o, _ = O.select_channels(p["X_warm"], 64)
    aw_o = O.compute_alpha(p["W"], idx_o)
    xo = O.quantize_nvfp4(p["X"], idx_o, ax_o)
    wo = O.quantize_nvfp4(p["W"][cols], idx_o, aw_o)
    Yo = O.splice_gemm(xo[0], xo[1], ax_o, xo[2], wo[0], wo[1], aw_o, wo[2])
    idx, ax, aw, gx, gw = gpu_packs(p["X_warm"], p["X"], p["W"], 64)
    Y = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
    Yn = S.nvfp4_gemm(gx[0], gx[1], ax, gw[0], gw[1], aw)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), idx_o) and scalar(aw) == np.float32(aw_o)
    assert np.array_equal(host(gx[0]), xo[0]) and np.array_equal(host(gw[0])[cols], wo[0])
    assert_gemm_close(host(Y)[:, cols], Yo, f"{name} M={M}")
    assert torch.isfinite(Yn).all()


@pytest.mark.parametrize("M", [700, 1024])
def test_prefill_mid_range_big_tile_sampled(M):
    """gate at 700 and 1024 rows: fewer than 240 tiles of 256 x 256, but more
    than one round of 128 x 128, so the big tile runs (ragged in the last
    tile row at 700): 160 sampled columns against the oracle's own
    calibration, packs and product."""
    p = synth.projection(synth.CFG_PREFILL, "gate", M)
    K, N = p["K"], p["N"]
    assert S.gemm_plan(M, N, K)[2:] == (256, 256, 1)
    cols = np.sort(np.random.default_rng(M + N).choice(N, size=160, replace=False))
    idx_o, ax_o, _ = O.select_channels(p["X_warm"], 64)
    aw_o = O.compute_alpha(p["W"], idx_o)
    xo = O.quantize_nvfp4(p["X"], idx_o, ax_o)
    wo = O.quantize_nvfp4(p["W"][cols], idx_o, aw_o)
    Yo = O.splice_gemm(xo[0], xo[1], ax_o, xo[2], wo[0], wo[1], aw_o, wo[2])
    idx, ax, aw, gx, gw = gpu_packs(p["X_warm"], p["X"], p["W"], 64)
    Y = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
    torch.cuda.synchronize()
    assert np.array_equal(host(gx[0]), xo[0]) and np.array_equal(host(gw[0])[cols], wo[0])
    assert_gemm_close(host(Y)[:, cols], Yo, f"gate M={M}")


# (M, N, K, k): ragged tiles in M and N, split counts that do not divide the
# K steps (K = 1664: 26 steps in splits of 9, 9, 8; K = 2176: 34 steps in
# 9, 9, 9, 7), many splits (K = 17408: 34; K = 12288: 24), every side-operand
# form (k = 0; 32 and 64 staged; 5 and 100 unaligned; 256 in two staged passes)
CASES = [(65, 64, 1024, 64), (100, 300, 1664, 5), (130, 250, 4096, 32), (200, 1000, 2176, 100),
         (77, 40, 17408, 16), (300, 129, 1152, 0), (96, 513, 4096, 256), (150, 128, 12288, 64)]


@pytest.mark.parametrize("M,N,K,k", CASES)
def test_split_prefill_ragged(M, N, K, k):
    g = np.random.default_rng(M * 7 + N + K + k)
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    ax, aw = np.float32(O.compute_alpha(X, idx)), np.float32(O.compute_alpha(W, idx))
    xq, xs, xS = O.quantize_nvfp4(X, idx, ax)
    wq, ws, wS = O.quantize_nvfp4(W, idx, aw)
    Yo = O.splice_gemm(xq, xs, ax, xS, wq, ws, aw, wS)
    assert S.gemm_plan(M, N, K)[4] > 1
    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    axd, awd = S.compute_alpha(Xd, idxd), S.compute_alpha(Wd, idxd)
    gx, gw = S.quantize_nvfp4(Xd, idxd, axd), S.quantize_nvfp4(Wd, idxd, awd)
    Y = S.splice_gemm(gx[0], gx[1], axd, gx[2] if k else None, gw[0], gw[1], awd, gw[2] if k else None)
    torch.cuda.synchronize()
    # the literal bar on every element
    assert_gemm_close(host(Y), Yo, f"M={M} N={N} K={K} k={k}")
    if k == 0:
        Yn = S.nvfp4_gemm(gx[0], gx[1], axd, gw[0], gw[1], awd)
        assert torch.equal(Yn, Y)


def test_split_prefill_repeat_and_shared_workspace():
    """Calls of three shapes take turns on one workspace: every call of a
    shape gives the first call's bits (the arrival counters return to zero,
    and the partials are summed in split order whatever the arrival order)."""
    g = np.random.default_rng(21)
    # more output tiles after fewer: the later call's counters must not land
    # on the earlier calls' partial tiles
    shapes = [(128, 1024, 4096), (200, 256, 12288), (65, 4096, 4096), (256, 4096, 12288)]
    ops = []
    for M, N, K in shapes:
        X = synth.to_bf16(g.standard_normal((M, K)))
        W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
        idx = dev(np.sort(g.choice(K, size=64, replace=False)).astype(np.int32))
        Xd, Wd = dev(X), dev(W)
        ax, aw = S.compute_alpha(Xd, idx), S.compute_alpha(Wd, idx)
        ops.append((S.quantize_nvfp4(Xd, idx, ax), S.quantize_nvfp4(Wd, idx, aw), ax, aw))
    ws = torch.zeros(max(S.workspace_size(*s) for s in shapes), dtype=torch.uint8, device="cuda")
    first = []
    for r in range(4):
        for i, (gx, gw, ax, aw) in enumerate(ops):
            Y = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], ws=ws)
            if r == 0:
                first.append(Y)
            else:
                torch.cuda.synchronize()
                assert torch.equal(Y, first[i]), f"round {r} shape {shapes[i]}"
    torch.cuda.synchronize()
    # the arrival counters (a fixed region of 256 slots at the front of the
    # workspace) are all back at zero
    assert int(ws[:1024].view(torch.int32).abs().sum().item()) == 0


def test_split_prefill_in_hip_graph():
    """A split call captured once and replayed with new activations in place
    (quantized eagerly between replays): every replay gives the eager call's
    bits."""
    g = np.random.default_rng(22)
    M, N, K, k = 128, 1024, 4096, 64
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    X0 = synth.to_bf16(g.standard_normal((M, K)))
    idx = dev(np.sort(g.choice(K, size=k, replace=False)).astype(np.int32))
    Xd, Wd = dev(X0), dev(W)
    ax, aw = S.compute_alpha(Xd, idx), S.compute_alpha(Wd, idx)
    gx, gw = S.quantize_nvfp4(Xd, idx, ax), S.quantize_nvfp4(Wd, idx, aw)
    Y = torch.empty(M, N, device="cuda")
    S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], out=Y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], out=Y)
    for r in range(3):
        X = synth.to_bf16(g.standard_normal((M, K)))
        S.quantize_nvfp4(dev(X), idx, ax, out=gx)
        graph.replay()
        torch.cuda.synchronize()
        ref = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), f"replay {r}"


# decode path, (M, N, K, k): every split form (1, 2 and 4 row blocks; 1, 2 and 4
# column blocks per group), ragged rows and columns, split counts that do not
# divide the chunks (K = 5248: 41 chunks in 9, 9, 9, 9, 5; K = 17408: 136 in
# 46, 46, 44), side operands k = 0, 32 and 64 (loaded ahead of the partial
# sums; W_S behind the first weight batch where each wave finishes a tile of
# its own, the 64 x 32 and 32 x 64 forms) and 5, 100, 256 (the general side
# loop)
DECODE_CASES = [(8, 1000, 8192, 32), (13, 1024, 4096, 64), (20, 500, 4608, 32), (29, 777, 5248, 5),
                (24, 4000, 12288, 64), (40, 1000, 4096, 64), (64, 4096, 12288, 0), (33, 2100, 17408, 100),
                (50, 64, 2048, 256), (48, 3000, 4096, 32), (30, 2000, 12288, 32)]


def oracle_case(M, N, K, k, seed):
    g = np.random.default_rng(seed)
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    return X, W, idx


@pytest.mark.parametrize("M,N,K,k", DECODE_CASES)
def test_split_decode_ragged(M, N, K, k):
    X, W, idx = oracle_case(M, N, K, k, M * 11 + N + K + k)
    ax, aw = np.float32(O.compute_alpha(X, idx)), np.float32(O.compute_alpha(W, idx))
    xq, xs, xS = O.quantize_nvfp4(X, idx, ax)
    wq, ws, wS = O.quantize_nvfp4(W, idx, aw)
    Yo = O.splice_gemm(xq, xs, ax, xS, wq, ws, aw, wS)
    plan = S.gemm_plan(M, N, K, S.PATH_DECODE)
    assert plan[0] == 1 and plan[4] > 1, plan
    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    axd, awd = S.compute_alpha(Xd, idxd), S.compute_alpha(Wd, idxd)
    gx, gw = S.quantize_nvfp4(Xd, idxd, axd), S.quantize_nvfp4(Wd, idxd, awd)
    args = (gx[0], gx[1], axd, gx[2] if k else None, gw[0], gw[1], awd, gw[2] if k else None)
    Y = S.splice_gemm(*args, path=S.PATH_DECODE)
    Y2 = S.splice_gemm(*args, path=S.PATH_DECODE)
    torch.cuda.synchronize()
    assert_gemm_close(host(Y), Yo, f"M={M} N={N} K={K} k={k} plan={plan}")
    assert torch.equal(Y, Y2)
    if k == 0:
        Yn = S.nvfp4_gemm(gx[0], gx[1], axd, gw[0], gw[1], awd, path=S.PATH_DECODE)
        assert torch.equal(Yn, Y)


def test_split_decode_shares_workspace_with_prefill():
    """Decode-path and prefill-path split calls take turns on one workspace:
    every call gives its first call's bits and the counters end at zero."""
    shapes = [(64, 1024, 4096, S.PATH_DECODE), (128, 1024, 4096, S.PATH_PREFILL),
              (24, 4000, 12288, S.PATH_DECODE), (8, 1000, 8192, S.PATH_DECODE),
              (65, 4096, 4096, S.PATH_PREFILL), (40, 4096, 4096, S.PATH_DECODE)]
    ops = []
    for i, (M, N, K, path) in enumerate(shapes):
        assert S.gemm_plan(M, N, K, path)[4] > 1
        X, W, idx = oracle_case(M, N, K, 64, 300 + i)
        Xd, Wd, idxd = dev(X), dev(W), dev(idx)
        ax, aw = S.compute_alpha(Xd, idxd), S.compute_alpha(Wd, idxd)
        ops.append((S.quantize_nvfp4(Xd, idxd, ax), S.quantize_nvfp4(Wd, idxd, aw), ax, aw, path))
    ws = torch.zeros(max(S.workspace_size(M, N, K) for M, N, K, _ in shapes), dtype=torch.uint8, device="cuda")
    first = []
    for r in range(3):
        for i, (gx, gw, ax, aw, path) in enumerate(ops):
            Y = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], path=path, ws=ws)
            if r == 0:
                first.append(Y)
            else:
                torch.cuda.synchronize()
                assert torch.equal(Y, first[i]), f"round {r} shape {shapes[i]}"
    torch.cuda.synchronize()
    assert int(ws[:1024].view(torch.int32).abs().sum().item()) == 0


def test_split_decode_in_hip_graph():
    """A decode-path split call (k at M = 32: four K ranges) captured once and
    replayed with new activations: every replay gives the eager call's bits."""
    M, N, K, k = 32, 1024, 4096, 64
    assert S.gemm_plan(M, N, K)[4] > 1
    X0, W, idx_h = oracle_case(M, N, K, k, 23)
    g = np.random.default_rng(24)
    idx = dev(idx_h)
    Xd, Wd = dev(X0), dev(W)
    ax, aw = S.compute_alpha(Xd, idx), S.compute_alpha(Wd, idx)
    gx, gw = S.quantize_nvfp4(Xd, idx, ax), S.quantize_nvfp4(Wd, idx, aw)
    Y = torch.empty(M, N, device="cuda")
    S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], out=Y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], out=Y)
    for r in range(3):
        X = synth.to_bf16(g.standard_normal((M, K)) * 2.0 ** r)
        S.quantize_nvfp4(dev(X), idx, ax, out=gx)
        graph.replay()
        torch.cuda.synchronize()
        ref = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), f"replay {r}"
