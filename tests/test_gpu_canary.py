"""Out-of-bounds write checks on the GPU: every GEMM form writes its output
into a view of a larger buffer filled with a sentinel (row stride ldy > N and
rows after the last one), and nothing outside the M x N product may change.
The product inside the view must equal the same call's contiguous output bit
for bit.  Shapes cover each kernel family with ragged edges in M and N: the
256 x 256 tile, the 128 x 128 tile unsplit and with its K range split over
workgroups, the decode forms, the multi-projection launch and the grouped
launch."""
import numpy as np
import pytest
import torch

from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu

SENTINEL = -12345.5
PAD_COLS, PAD_ROWS = 40, 8


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def packs(M, N, K, k, seed):
    g = np.random.default_rng(seed)
    X = synth.to_bf16(g.standard_normal((M, K)))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = dev(np.sort(g.choice(K, size=k, replace=False)).astype(np.int32))
    Xd, Wd = dev(X), dev(W)
    ax, aw = S.compute_alpha(Xd, idx), S.compute_alpha(Wd, idx)
    return S.quantize_nvfp4(Xd, idx, ax), S.quantize_nvfp4(Wd, idx, aw), ax, aw


def padded(M, N):
    big = torch.full((M + PAD_ROWS, N + PAD_COLS), SENTINEL, device="cuda")
    return big, big[:M, :N]


def untouched(big, M, N):
    b = big.cpu()
    return bool((b[:M, N:] == SENTINEL).all() and (b[M:, :] == SENTINEL).all())


# (M, N, K, k, path): 256 x 256 tiles with ragged edges, 128 x 128 unsplit,
# 128 x 128 with the K range split, decode unsplit, decode with the K range
# split (1, 2 and 4 row blocks)
CASES = [(4000, 4000, 256, 64, S.PATH_PREFILL), (2000, 1100, 512, 64, S.PATH_PREFILL),
         (100, 300, 1664, 64, S.PATH_PREFILL), (130, 250, 4096, 32, S.PATH_PREFILL),
         (37, 1000, 1024, 64, S.PATH_DECODE), (3, 8200, 384, 64, S.PATH_DECODE),
         (64, 520, 12288, 16, S.PATH_DECODE), (8, 1000, 8192, 32, S.PATH_DECODE),
         (24, 4000, 12288, 64, S.PATH_DECODE), (40, 1000, 4096, 64, S.PATH_DECODE)]


@pytest.mark.parametrize("M,N,K,k,path", CASES)
def test_gemm_writes_only_its_product(M, N, K, k, path):
    gx, gw, ax, aw = packs(M, N, K, k, M + N + K)
    ref = S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], path=path)
    big, view = padded(M, N)
    S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], path=path, out=view)
    torch.cuda.synchronize()
    assert torch.equal(view, ref), (M, N, K, k, path, S.gemm_plan(M, N, K, path))
    assert untouched(big, M, N), (M, N, K, k, path, S.gemm_plan(M, N, K, path))


@pytest.mark.parametrize("M,K,path", [(300, 1024, S.PATH_PREFILL), (96, 1024, S.PATH_PREFILL),
                                      (8, 1024, S.PATH_DECODE), (8, 4096, S.PATH_DECODE),
                                      (40, 4096, S.PATH_DECODE)])
def test_multi_writes_only_its_products(M, K, path):
    k, widths = 64, [520, 136, 136]
    gx, _, ax, _ = packs(M, 8, K, k, 7 + M)
    weights = []
    for i, n in enumerate(widths):
        _, gw, _, aw = packs(8, n, K, k, 100 + i)
        weights.append((gw[0], gw[1], aw, gw[2]))
    refs = S.splice_gemm_multi(gx[0], gx[1], ax, gx[2], weights, path=path)
    bigs = [padded(M, n) for n in widths]
    S.splice_gemm_multi(gx[0], gx[1], ax, gx[2], weights, path=path, out=[v for _, v in bigs])
    torch.cuda.synchronize()
    for (big, view), ref, n in zip(bigs, refs, widths):
        assert torch.equal(view, ref), (M, n)
        assert untouched(big, M, n), (M, n)


def test_grouped_writes_only_its_products():
    K, N, k = 512, 200, 16
    Ms = [0, 1, 70, 128, 129, 300]
    groups, refs, bigs = [], [], []
    for e, Me in enumerate(Ms):
        gx, gw, ax, aw = packs(max(Me, 1), N, K, k, 50 + e)
        gx = tuple(t[:Me] for t in gx)
        big, view = padded(Me, N)
        groups.append(dict(Xq=gx[0], Xs=gx[1], alpha_x=ax, X_S=gx[2], Wq=gw[0], Ws=gw[1], alpha_w=aw,
                           W_S=gw[2], Y=view))
        bigs.append(big)
        refs.append(S.splice_gemm(gx[0], gx[1], ax, gx[2], gw[0], gw[1], aw, gw[2], path=S.PATH_PREFILL)
                    if Me else None)
    # the grouped form writes with ldy = N: give each group a contiguous view
    # of exactly M x N inside its padded buffer's first rows
    for grp, big, Me in zip(groups, bigs, Ms):
        grp["Y"] = big.view(-1)[:Me * N].view(Me, N) if Me else big[:0, :N]
    S.splice_gemm_grouped(groups, N, K, k)
    torch.cuda.synchronize()
    for e, (grp, big, Me) in enumerate(zip(groups, bigs, Ms)):
        flat = big.view(-1)
        assert bool((flat[Me * N:] == SENTINEL).all()), f"group {e} M={Me}"
        if Me:
            assert torch.equal(grp["Y"], refs[e]), f"group {e} M={Me}"
