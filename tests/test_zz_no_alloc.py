"""splice_gemm_noalloc on the GPU, through the C ABI: the allocation-free
entry point (its workspace is the library's own per-device array) gives
splice_gemm's bits, for two calls in a row on the K-split prefill path, the
second smaller, and decode-path calls after them, with and without a K
split."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth
from gpu_util import assert_gemm_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def packs(M, N, K, k, seed):
    g = np.random.default_rng(seed)
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    ax, aw = S.compute_alpha(Xd, idxd), S.compute_alpha(Wd, idxd)
    return S.quantize_nvfp4(Xd, idxd, ax), S.quantize_nvfp4(Wd, idxd, aw), ax, aw, (X, W, idx)


def test_noalloc_matches_splice_gemm_two_calls():
    # (M, N, K, k): a K-split prefill call, a smaller one (fewer tiles, a
    # different split count), a decode-path call with its K range split, and
    # one that needs no workspace
    cases = [(200, 1000, 4096, 64), (96, 300, 2176, 64), (40, 1000, 4096, 64), (8, 512, 1024, 64)]
    for i, (M, N, K, k) in enumerate(cases):
        gx, gw, ax, aw, (X, W, idx) = packs(M, N, K, k, 31 + i)
        assert (S.gemm_plan(M, N, K)[4] > 1) == (i < 3)
        Y_ref = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
        Y = torch.full((M, N), float("nan"), device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        S.splice_gemm_noalloc(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], out=Y)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert_gemm_close(host(Y), host(Y_ref).astype(np.float64), f"M={M} N={N} K={K} vs splice_gemm")
        assert torch.equal(Y, Y_ref), f"M={M} N={N} K={K}: bits differ from splice_gemm"
        # and the oracle's product on the same operands
        axo, awo = np.float32(ax.item()), np.float32(aw.item())
        xo, wo = O.quantize_nvfp4(X, idx, axo), O.quantize_nvfp4(W, idx, awo)
        cols = np.arange(0, N, 7)
        Yo = O.splice_gemm(xo[0], xo[1], axo, xo[2], wo[0][cols], wo[1][cols], awo, wo[2][cols])
        assert_gemm_close(host(Y)[:, cols], Yo, f"M={M} N={N} K={K} vs oracle")


def test_noalloc_repeated_calls_keep_bits():
    """The array keeps the last call's contents; its counters return to zero,
    so the same call repeated gives the same bits."""
    gx, gw, ax, aw, _ = packs(130, 700, 4096, 64, 40)
    Y0 = S.splice_gemm_noalloc(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
    for _ in range(3):
        Y = S.splice_gemm_noalloc(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2])
        torch.cuda.synchronize()
        assert torch.equal(Y, Y0)
