"""GPU parity at one rank's shapes under 8-way tensor parallelism (Qwen3-8B
projections, rank 0), through the C ABI.

Column-parallel q, k and gate hold N/8 rows of W and the whole X;
row-parallel o and down hold K/8 channels of X and W, with the protected
channels that fall among them (a row-parallel rank's Y is a partial sum that
an all-reduce adds).  The protected set and both tensor scales are the whole
layer's: the GPU computes them on the full tensors, the oracle on its own.
Each rank's packs and product are compared with the oracle's on the same
shard: packs bit-exact, Y to the GEMM tolerance (every element at 1 and 64
rows; 96 sampled columns of all 8192 rows).
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth
from gpu_util import assert_gemm_close, dev, host, scalar

pytestmark = pytest.mark.gpu

TP = 8
SHARDS = [("q", "col"), ("k", "col"), ("gate", "col"), ("o", "row"), ("down", "row")]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.mark.parametrize("M", [1, 64, 8192])
@pytest.mark.parametrize("name,kind", SHARDS)
def test_tp8_rank_shard(name, kind, M):
    p = synth.projection(synth.CFG_PREFILL, name, M)
    K, N = p["K"], p["N"]
    X, W, Xw = p["X"], p["W"], p["X_warm"]
    # the layer's protected set and tensor scales, on the full tensors
    idx_o, ax_o, _ = O.select_channels(Xw, 64)
    aw_o = O.compute_alpha(W, idx_o)
    Xwd, Xd, Wd = dev(Xw), dev(X), dev(W)
    idx, ax, _ = S.select_channels(Xwd, 64)
    aw = S.compute_alpha(Wd, idx)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), idx_o) and scalar(aw) == np.float32(aw_o)
    if kind == "col":
        Kr, Nr = K, N // TP
        Xs_o, Ws_o, il_o = X, W[:Nr], idx_o
        Xs_d, Ws_d, il_d = Xd, Wd[:Nr], idx
    else:
        Kr, Nr = K // TP, N
        Xs_o, Ws_o = np.ascontiguousarray(X[:, :Kr]), np.ascontiguousarray(W[:, :Kr])
        il_o = idx_o[idx_o < Kr]
        Xs_d, Ws_d = Xd[:, :Kr], Wd[:, :Kr]           # strided views (row stride K)
        il_d = idx[idx < Kr].contiguous()
    kr = len(il_o)
    assert int(il_d.numel()) == kr
    cols = np.arange(Nr) if M <= 64 else np.sort(np.random.default_rng(M + Nr).choice(Nr, 96, replace=False))
    xo = O.quantize_nvfp4(Xs_o, il_o, np.float32(ax_o))
    wo = O.quantize_nvfp4(Ws_o[cols], il_o, np.float32(aw_o))
    Yo = O.splice_gemm(xo[0], xo[1], ax_o, xo[2] if kr else None, wo[0], wo[1], aw_o, wo[2] if kr else None)
    gx = S.quantize_nvfp4(Xs_d, il_d, ax)
    gw = S.quantize_nvfp4(Ws_d, il_d, aw)
    Y = S.splice_gemm(gx[0], gx[1], ax, gx[2] if kr else None, gw[0], gw[1], aw, gw[2] if kr else None)
    torch.cuda.synchronize()
    assert np.array_equal(host(gx[0]), xo[0]) and np.array_equal(host(gx[1]), xo[1])
    assert np.array_equal(host(gw[0])[cols], wo[0]) and np.array_equal(host(gw[1])[cols], wo[1])
    if kr:
        assert np.array_equal(host(gx[2]), xo[2])
    assert_gemm_close(host(Y)[:, cols], Yo, f"{name} {kind} rank shard K={Kr} N={Nr} k={kr} M={M} "
                      f"plan={S.gemm_plan(M, Nr, Kr)}")
