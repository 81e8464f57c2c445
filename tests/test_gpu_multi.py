"""GPU parity of splice_gemm_multi, one launch over several weight matrices
that share the activation operands, through the C ABI.

Against separate splice_gemm calls on the same packs: bit-identical wherever
the launch's plan (tile and K split, splice_multi_plan) is the plan each call
alone makes (splice_gemm_plan), within the GEMM tolerance elsewhere.  Against
the oracle: the tolerance in gpu_util, segment by segment.
"""
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


def packs(X, Ws, k, seed):
    """Device packs of X and of each weight matrix, with X's top-k channels
    from a warm-up batch drawn like X."""
    Xw = dev(synth.activations(7, seed % 4, 256, X.shape[1], 2 + 10 * seed, "student", n_out=8))
    idx, ax, _ = S.select_channels(Xw, k)
    xq = S.quantize_nvfp4(dev(X), idx, ax)
    wp = []
    for W in Ws:
        Wd = dev(W)
        aw = S.compute_alpha(Wd, idx)
        wq = S.quantize_nvfp4(Wd, idx, aw)
        wp.append((wq[0], wq[1], aw, wq[2] if k else None))
    packs.idx = idx
    return xq, ax, wp


def separate(xq, ax, wp, k, path):
    return [S.splice_gemm(xq[0], xq[1], ax, xq[2] if k else None, *w, path=path) for w in wp]


def same_plan(M, K, widths, path):
    """True when one launch over these widths runs the arithmetic each call
    alone runs: the same path, kernel and K split (the tile size of the
    prefill path does not change the summation order)."""
    key = lambda p: (p[0], p[1], p[4])
    mp = key(S.multi_plan(M, K, widths, path))
    return all(key(S.gemm_plan(M, n, K, path)) == mp for n in widths if n > 0)


@pytest.mark.parametrize("M", [1, 3, 8, 20, 40, 64, 100, 300])
@pytest.mark.parametrize("k", [0, 8, 64])
def test_ragged_segments(M, k):
    """Five segments of ragged widths (one empty) against separate calls and
    the oracle; K = 1024."""
    check_ragged_segments(M, k, 1024)


@pytest.mark.parametrize("M", [8, 20, 40, 64, 100])
@pytest.mark.parametrize("k", [0, 64])
def test_ragged_segments_split_k(M, k):
    """The same five segments at K = 4096, where the launch splits its K range
    over workgroups on either path (column groups or tiles counted per
    segment)."""
    assert S.multi_plan(M, 4096, [100, 17, 0, 300, 64])[4] > 1
    check_ragged_segments(M, k, 4096)


def check_ragged_segments(M, k, K):
    widths = [100, 17, 0, 300, 64]
    g = np.random.default_rng(M * 10 + k + (0 if K == 1024 else K))
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    Ws = [synth.to_bf16(g.normal(0, 0.02, (n, K))) for n in widths]
    xq, ax, wp = packs(X, Ws, k, M + k)
    path = S.PATH_AUTO
    Ym = S.splice_gemm_multi(xq[0], xq[1], ax, xq[2] if k else None, wp, path=path)
    Yd = separate(xq, ax, wp, k, path)
    torch.cuda.synchronize()
    exact = same_plan(M, K, widths, path)
    xo = (host(xq[0]), host(xq[1]), np.float32(ax.item()), host(xq[2]))
    for i, (a, b) in enumerate(zip(Ym, Yd)):
        assert a.shape == (M, widths[i])
        if exact:
            assert torch.equal(a, b), f"segment {i}"
        if widths[i] == 0:
            continue
        wo = (host(wp[i][0]), host(wp[i][1]), np.float32(wp[i][2].item()),
              host(wp[i][3]) if k else np.zeros((widths[i], 0), np.uint16))
        Yo = O.splice_gemm(xo[0], xo[1], xo[2], xo[3] if k else None, wo[0], wo[1], wo[2],
                           wo[3] if k else None)
        assert_gemm_close(host(a), Yo, f"M={M} k={k} segment {i}")


@pytest.mark.parametrize("M", [1, 8, 32, 64, 512, 8192])
@pytest.mark.parametrize("group", ["qkv", "gate_up"])
def test_layer_groups_bit_identical(M, group):
    """The projections that read one Qwen3-8B layer input, in one launch, give
    the separate calls' bits where the plans agree -- gate and up at every M,
    q, k and v at M = 1 and 8192, the timed step's size (the separate calls
    meet the oracle at that size in test_gpu_parity) -- and agree to the
    tolerance where the K split differs (q, k and v at M = 8..64 and 512:
    alone, k and v split their sums, and q at M = 64, where the launch of all
    three does not, or fewer ways)."""
    names = ["q", "k", "v"] if group == "qkv" else ["gate", "up"]
    K = synth.QWEN3_8B[names[0]][0]
    g = np.random.default_rng(5)
    X = synth.activations(synth.CFG_DECODE, 0, M, K, 3, "student")
    Ws = [synth.to_bf16(g.normal(0, 0.02, (synth.QWEN3_8B[n][1], K))) for n in names]
    xq, ax, wp = packs(X, Ws, 64, 1)
    Ym = S.splice_gemm_multi(xq[0], xq[1], ax, xq[2], wp)
    Yd = separate(xq, ax, wp, 64, S.PATH_AUTO)
    torch.cuda.synchronize()
    widths = [synth.QWEN3_8B[n][1] for n in names]
    exact = same_plan(M, K, widths, S.PATH_AUTO)
    assert exact == (group == "gate_up" or M in (1, 8192)), (M, S.multi_plan(M, K, widths),
                                                        [S.gemm_plan(M, w, K) for w in widths])
    for n, a, b in zip(names, Ym, Yd):
        if exact:
            assert torch.equal(a, b), f"{group} M={M}: {n}"
        else:
            assert_gemm_close(host(a), host(b).astype(np.float64), f"{group} M={M}: {n}")


def test_output_row_stride_and_forced_paths():
    """Outputs that are column slices of one wider buffer (ldy > N), on both
    paths."""
    M, K, widths = 24, 512, [48, 80]
    g = np.random.default_rng(3)
    X = synth.to_bf16(g.standard_normal((M, K)))
    Ws = [synth.to_bf16(g.normal(0, 0.02, (n, K))) for n in widths]
    xq, ax, wp = packs(X, Ws, 8, 3)
    for path in (S.PATH_DECODE, S.PATH_PREFILL):
        buf = torch.full((M, 200), float("nan"), device="cuda")
        outs = [buf[:, 0:48], buf[:, 60:140]]
        S.splice_gemm_multi(xq[0], xq[1], ax, xq[2], wp, path=path, out=outs)
        Yd = separate(xq, ax, wp, 8, path)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], Yd[0]) and torch.equal(outs[1], Yd[1])
        assert torch.isnan(buf[:, 48:60]).all() and torch.isnan(buf[:, 140:]).all()


def test_multi_in_hip_graph():
    """Captured once and replayed with new activations in place: every replay
    equals the eager call."""
    M, K, widths = 4, 1024, [256, 64, 64]
    g = np.random.default_rng(8)
    Ws = [synth.to_bf16(g.normal(0, 0.02, (n, K))) for n in widths]
    X0 = synth.to_bf16(g.standard_normal((M, K)))
    xq, ax, wp = packs(X0, Ws, 64, 8)
    idx = packs.idx
    outs = [torch.empty(M, n, device="cuda") for n in widths]
    S.splice_gemm_multi(xq[0], xq[1], ax, xq[2], wp, out=outs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        S.splice_gemm_multi(xq[0], xq[1], ax, xq[2], wp, out=outs)
    for r in range(3):
        X = synth.to_bf16(g.standard_normal((M, K)))
        S.quantize_nvfp4(dev(X), idx, ax, out=xq)
        graph.replay()
        torch.cuda.synchronize()
        ref = S.splice_gemm_multi(xq[0], xq[1], ax, xq[2], wp)
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r}"


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("group", ["qkv", "gate_up"])
def test_fused_prep_layer_groups(M, group):
    """The fused-preparation decode over the projections of one input: the
    bits of splice_gemm_decode_fused per projection (the combined width only
    changes how columns are grouped into workgroups), and the oracle's product
    on sampled columns."""
    names = ["q", "k", "v"] if group == "qkv" else ["gate", "up"]
    K = synth.QWEN3_8B[names[0]][0]
    g = np.random.default_rng(9)
    X = synth.activations(synth.CFG_DECODE, 0, M, K, 3, "student")
    Ws = [synth.to_bf16(g.normal(0, 0.02, (synth.QWEN3_8B[n][1], K))) for n in names]
    xq, ax, wp = packs(X, Ws, 64, 2)
    idx = packs.idx
    Xd = dev(X)
    Ym = S.splice_gemm_decode_fused_multi(Xd, idx, ax, wp)
    Yf = [S.splice_gemm_decode_fused(Xd, idx, ax, *w) for w in wp]
    torch.cuda.synchronize()
    xo = O.quantize_nvfp4(X, host(idx), np.float32(ax.item()))
    for i, (n, a, b) in enumerate(zip(names, Ym, Yf)):
        widths = [w[0].shape[0] for w in wp]
        assert torch.equal(a, b), f"{group} M={M}: {n}"
        cols = np.arange(0, widths[i], 97)
        wq, ws, aw, wS = (host(wp[i][0])[cols], host(wp[i][1])[cols], np.float32(wp[i][2].item()),
                          host(wp[i][3])[cols])
        Yo = O.splice_gemm(xo[0], xo[1], np.float32(ax.item()), xo[2], wq, ws, aw, wS)
        assert_gemm_close(host(a)[:, cols], Yo, f"{group} M={M}: {n} vs oracle")


def test_fused_prep_ragged_segments():
    """Ragged widths, one empty, K = 256 and 1024, and K = 12288 (sixteen
    waves of six chunks), against the per-segment fused call."""
    g = np.random.default_rng(4)
    for M, K in ((1, 256), (3, 1024), (4, 1024), (2, 12288), (4, 12288)):
        widths = [40, 0, 130, 16]
        X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
        Ws = [synth.to_bf16(g.normal(0, 0.02, (n, K))) for n in widths]
        xq, ax, wp = packs(X, Ws, 8, 5)
        idx = packs.idx
        Xd = dev(X)
        Ym = S.splice_gemm_decode_fused_multi(Xd, idx, ax, wp)
        Yf = [S.splice_gemm_decode_fused(Xd, idx, ax, *w) for w in wp]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(Ym, Yf)):
            assert a.shape == (M, widths[i])
            assert torch.equal(a, b), f"M={M} K={K} segment {i}"


def test_fused_prep_combined_width_crosses_wide_form():
    """Two segments of 256 and 257 column blocks: alone each takes 16 columns
    per workgroup, together (513 blocks) the 48-column form; the bits do not
    change."""
    g = np.random.default_rng(6)
    M, K, widths = 2, 1024, [4096, 4100]
    X = synth.to_bf16(g.standard_normal((M, K)))
    Ws = [synth.to_bf16(g.normal(0, 0.02, (n, K))) for n in widths]
    xq, ax, wp = packs(X, Ws, 64, 6)
    idx = packs.idx
    Xd = dev(X)
    Ym = S.splice_gemm_decode_fused_multi(Xd, idx, ax, wp)
    Yf = [S.splice_gemm_decode_fused(Xd, idx, ax, *w) for w in wp]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(Ym, Yf)):
        assert torch.equal(a, b), f"segment {i}"
