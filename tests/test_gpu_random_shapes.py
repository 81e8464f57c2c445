"""GPU parity on seeded random shapes across every plan: M from 1 to 3000
(decode forms with and without a K split, the 128 x 128 tile with and
without one, the 256 x 256 tile), N up to 9000, K up to 12672, k from 0 to
256, each path the shape allows.  Sampled rows and columns of every product
against the oracle's, to the GEMM tolerance, and a repeated call bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth
from gpu_util import assert_gemm_close, dev, host

pytestmark = pytest.mark.gpu

M_CHOICES = [1, 2, 3, 4, 5, 8, 13, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 128, 200, 257, 511, 512, 513,
             700, 1024, 1500, 2100, 3000]


def random_case(c):
    r = np.random.default_rng(7000 + c)
    M = int(r.choice(M_CHOICES))
    N = int(r.integers(1, 9000))
    K = 128 * int(r.integers(1, 100))
    k = min(int(r.choice([0, 1, 5, 8, 31, 32, 64, 100, 256])), K)
    paths = [S.PATH_AUTO, S.PATH_PREFILL] + ([S.PATH_DECODE] if M <= S.DECODE_MAX_M else [])
    path = int(r.choice(paths))
    if M * K > 3000 * 8000:                 # keep each case within a second or two
        K = 128 * max(1, (3000 * 8000 // M) // 128)
    return M, N, K, k, path


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.mark.parametrize("c", range(60))
def test_random_shape(c):
    M, N, K, k, path = random_case(c)
    g = np.random.default_rng(c)
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    rows = np.sort(g.choice(M, size=min(M, 24), replace=False))
    cols = np.sort(g.choice(N, size=min(N, 48), replace=False))
    ax, aw = np.float32(O.compute_alpha(X, idx)), np.float32(O.compute_alpha(W, idx))
    xq, xs, xS = O.quantize_nvfp4(X[rows], idx, ax)
    wq, ws, wS = O.quantize_nvfp4(W[cols], idx, aw)
    Yo = O.splice_gemm(xq, xs, ax, xS, wq, ws, aw, wS)
    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    axd, awd = S.compute_alpha(Xd, idxd), S.compute_alpha(Wd, idxd)
    gx, gw = S.quantize_nvfp4(Xd, idxd, axd), S.quantize_nvfp4(Wd, idxd, awd)
    args = (gx[0], gx[1], axd, gx[2] if k else None, gw[0], gw[1], awd, gw[2] if k else None)
    Y = S.splice_gemm(*args, path=path)
    Y2 = S.splice_gemm(*args, path=path)
    torch.cuda.synchronize()
    what = f"M={M} N={N} K={K} k={k} path={path} plan={S.gemm_plan(M, N, K, path)}"
    assert torch.equal(Y, Y2), what
    assert_gemm_close(host(Y)[np.ix_(rows, cols)], Yo, what)
