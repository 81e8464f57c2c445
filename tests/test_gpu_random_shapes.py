"""GPU parity on seeded random shapes across every plan: M from 1 to 3000
(decode forms with and without a K split, the 128 x 128 tile with and
without one, the 256 x 256 tile), N up to 9000, K up to 12672, k from 0 to
256, each path the shape allows; the multi-projection launch over random
segment widths; the fused-preparation decode at 1 to 4 rows.  Sampled rows
and columns of every product against the oracle's, to the GEMM tolerance,
and a repeated call bit for bit.
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


def random_packs(g, M, K, k, widths):
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    Ws = [synth.to_bf16(g.normal(0, 0.02, (n, K))) for n in widths]
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    return X, Ws, idx


@pytest.mark.parametrize("c", range(30))
def test_random_multi(c):
    """splice_gemm_multi over 1 to 8 segments of random widths (some empty)
    on either allowed path: every segment's sampled outputs against the
    oracle and a repeated launch bit for bit."""
    r = np.random.default_rng(8000 + c)
    M = int(r.choice(M_CHOICES))
    K = 128 * int(r.integers(1, 64))
    k = min(int(r.choice([0, 5, 32, 64, 100])), K)
    nseg = int(r.integers(1, S.SEG_MAX + 1))
    widths = [int(w) if r.random() > 0.15 else 0 for w in r.integers(1, 3000, nseg)]
    if not any(widths):
        widths[0] = 17
    paths = [S.PATH_AUTO, S.PATH_PREFILL] + ([S.PATH_DECODE] if M <= S.DECODE_MAX_M else [])
    path = int(r.choice(paths))
    g = np.random.default_rng(c)
    X, Ws, idx = random_packs(g, M, K, k, widths)
    rows = np.sort(g.choice(M, size=min(M, 16), replace=False))
    ax = np.float32(O.compute_alpha(X, idx))
    xo = O.quantize_nvfp4(X[rows], idx, ax)
    Xd, idxd = dev(X), dev(idx)
    axd = S.compute_alpha(Xd, idxd)
    gx = S.quantize_nvfp4(Xd, idxd, axd)
    weights, refs = [], []
    for W in Ws:
        n = W.shape[0]
        aw = np.float32(O.compute_alpha(W, idx)) if n else np.float32(1.0)
        cols = np.sort(g.choice(n, size=min(n, 32), replace=False)) if n else np.zeros(0, np.int64)
        if n:
            wo = O.quantize_nvfp4(W[cols], idx, aw)
            refs.append((cols, O.splice_gemm(xo[0], xo[1], ax, xo[2], wo[0], wo[1], aw, wo[2])))
        else:
            refs.append(None)
        Wd = dev(W) if n else torch.zeros(0, K, dtype=torch.int16, device="cuda")
        awd = S.compute_alpha(Wd, idxd) if n else dev(np.array([1.0], np.float32))
        gw = S.quantize_nvfp4(Wd, idxd, awd)
        weights.append((gw[0], gw[1], awd, gw[2] if k else None))
    Ys = S.splice_gemm_multi(gx[0], gx[1], axd, gx[2] if k else None, weights, path=path)
    Ys2 = S.splice_gemm_multi(gx[0], gx[1], axd, gx[2] if k else None, weights, path=path)
    torch.cuda.synchronize()
    what = f"M={M} K={K} k={k} widths={widths} path={path} plan={S.multi_plan(M, K, widths, path)}"
    for i, (Y, Y2, ref) in enumerate(zip(Ys, Ys2, refs)):
        assert torch.equal(Y, Y2), f"{what} segment {i}"
        if ref is not None:
            cols, Yo = ref
            assert_gemm_close(host(Y)[np.ix_(rows, cols)], Yo, f"{what} segment {i}")


@pytest.mark.parametrize("c", range(20))
def test_random_fused_decode(c):
    """splice_gemm_decode_fused at 1 to 4 rows on random N, K and k within
    its limits (K a multiple of 128 up to 16384, the FP16 rows within 128 KB):
    sampled outputs against the oracle's own quantization and product, and a
    repeated call bit for bit."""
    r = np.random.default_rng(9000 + c)
    M = int(r.integers(1, S.FUSED_MAX_M + 1))
    N = int(r.integers(1, 9000))
    K = 128 * int(r.integers(1, 129))
    k = min(int(r.choice([0, 5, 32, 64, 200])), K)
    g = np.random.default_rng(c)
    X, Ws, idx = random_packs(g, M, K, k, [N])
    W = Ws[0]
    cols = np.sort(g.choice(N, size=min(N, 48), replace=False))
    ax, aw = np.float32(O.compute_alpha(X, idx)), np.float32(O.compute_alpha(W, idx))
    xo = O.quantize_nvfp4(X, idx, ax)
    wo = O.quantize_nvfp4(W[cols], idx, aw)
    Yo = O.splice_gemm(xo[0], xo[1], ax, xo[2], wo[0], wo[1], aw, wo[2])
    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    axd, awd = dev(np.array([ax], np.float32)), S.compute_alpha(Wd, idxd)
    gw = S.quantize_nvfp4(Wd, idxd, awd)
    args = (Xd, idxd if k else None, axd, gw[0], gw[1], awd, gw[2] if k else None)
    Y = S.splice_gemm_decode_fused(*args)
    Y2 = S.splice_gemm_decode_fused(*args)
    torch.cuda.synchronize()
    what = f"M={M} N={N} K={K} k={k}"
    assert torch.equal(Y, Y2), what
    assert_gemm_close(host(Y)[:, cols], Yo, what)
