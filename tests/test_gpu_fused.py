"""GPU parity of the decode GEMM with the activation preparation fused into it
(splice_gemm_decode_fused) through the C ABI.

Against the oracle: the tolerance in gpu_util, with the oracle quantizing the
bf16 activations itself.  Against the two-call form (splice_quantize_nvfp4,
then splice_gemm on the decode path): bit-identical wherever the two-call form
runs its activations-in-LDS kernel with the fused call's wave configuration
(same_kernel below), since the same FP16 operands then enter the same
matrix-core sequence and the same summation order; elsewhere the two forms sum
the K chunks in different orders and agree to the tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth
from gpu_util import assert_gemm_close, dev, host, scalar

pytestmark = pytest.mark.gpu

XLDS_BYTES = 64 * 1024     # FP16 activations the two-call decode keeps in LDS


def same_kernel(M, K):
    """The two-call decode runs the kernel the fused call mirrors, with the
    same waves: an even chunk count and X in its LDS budget."""
    nchunk = K // 128
    return M * K * 2 <= XLDS_BYTES and nchunk % 2 == 0


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def two_call(Xd, idxd, axd, wq, ws, awd, wS, k):
    xq, xs, xS = S.quantize_nvfp4(Xd, idxd, axd)
    return S.splice_gemm(xq, xs, axd, xS if k else None, wq, ws, awd, wS if k else None,
                         path=S.PATH_DECODE)


def check_case(X, W, idx, what, ldx_pad=0):
    M, K = X.shape
    k = len(idx)
    ax, aw = np.float32(O.compute_alpha(X, idx)), np.float32(O.compute_alpha(W, idx))
    xq, xs, xS = O.quantize_nvfp4(X, idx, ax)
    wq_o, ws_o, wS_o = O.quantize_nvfp4(W, idx, aw)
    Yo = O.splice_gemm(xq, xs, ax, xS, wq_o, ws_o, aw, wS_o)

    if ldx_pad:
        Xbig = np.zeros((M, K + ldx_pad), np.uint16)
        Xbig[:, :K] = X
        Xd = dev(Xbig)[:, :K]
    else:
        Xd = dev(X)
    Wd, idxd = dev(W), dev(idx)
    axd = torch.tensor([ax], device="cuda")
    awd = S.compute_alpha(Wd, idxd)
    assert scalar(awd) == aw
    wq, ws, wS = S.quantize_nvfp4(Wd, idxd, awd)
    Yf = S.splice_gemm_decode_fused(Xd, idxd if k else None, axd, wq, ws, awd, wS if k else None)
    Y2 = two_call(Xd, idxd, axd, wq, ws, awd, wS, k)
    torch.cuda.synchronize()
    assert_gemm_close(host(Yf), Yo, what)
    if same_kernel(M, K):
        assert torch.equal(Yf, Y2), f"{what}: fused and two-call results differ"
    else:
        assert_gemm_close(host(Yf), host(Y2).astype(np.float64), what + " vs two-call")


# (M, N, K, k): several 16-column blocks and a ragged tail in N, every wave
# count of the dispatch (K up to 32, 64, 96, 128 chunks; odd chunk counts),
# 48-column workgroups for wide N (N >= 8192 with K <= 4096), the side-operand
# forms (k = 0; 32 and 64 preloaded; ragged, unaligned and all-protected)
CASES = [(1, 16, 256, 0), (1, 100, 1024, 5), (2, 48, 512, 64), (3, 130, 1024, 32),
         (4, 1000, 1024, 64), (1, 272, 4096, 64), (4, 80, 4096, 100), (2, 70, 8192, 33),
         (1, 50, 12288, 64), (4, 40, 12288, 64), (3, 24, 16384, 16), (1, 33, 16384, 128),
         (2, 64, 256, 256), (4, 17, 768, 7), (1, 40, 128, 16), (3, 60, 384, 64),
         (2, 90, 1152, 0), (1, 8200, 1024, 64), (2, 8195, 512, 5), (4, 8240, 4096, 32),
         (1, 8192, 640, 0), (3, 8210, 2048, 64), (3, 8192, 4096, 0)]


@pytest.mark.parametrize("M,N,K,k", CASES)
def test_fused_decode_shapes(M, N, K, k):
    g = np.random.default_rng(7000 + M * 100 + K + k)
    X = synth.to_bf16(g.standard_normal((M, K)) * np.where(g.random(K) < 0.03, 30.0, 1.0))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    check_case(X, W, idx, f"M={M} N={N} K={K} k={k}")


def test_fused_decode_special_values_and_row_stride():
    """Rows of zeros, negative zeros, tiny and huge values, with X read
    through a row stride larger than K."""
    g = np.random.default_rng(77)
    M, N, K, k = 4, 64, 1024, 48
    X = synth.to_bf16(g.standard_normal((M, K)))
    X[1] = 0x8000                                          # -0 everywhere
    X[2, ::3] = synth.to_bf16(np.full(K, 1e-30))[::3]      # tiny values
    X[3, ::5] = synth.to_bf16(np.full(K, 3e4))[::5]        # large values
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    check_case(X, W, idx, "special rows, ldx = K + 40", ldx_pad=40)


def test_fused_decode_tiny_tensor():
    """A tensor so small that alpha < 2^-80: the quantizer's fp64 threshold
    arithmetic (the fp32 form needs alpha >= 2^-80)."""
    g = np.random.default_rng(80)
    M, N, K, k = 3, 96, 512, 16
    X = synth.to_bf16(g.standard_normal((M, K)) * 1e-30)
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.sort(g.choice(K, size=k, replace=False)).astype(np.int32)
    assert O.compute_alpha(X, idx) < 2.0 ** -80
    check_case(X, W, idx, "tiny tensor")


def test_fused_decode_output_stride_and_empty_k():
    g = np.random.default_rng(78)
    M, N, K, k = 2, 64, 512, 16
    X = synth.to_bf16(g.standard_normal((M, K)))
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    idx = np.arange(0, K, K // k, dtype=np.int32)
    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    axd, awd = S.compute_alpha(Xd, idxd), S.compute_alpha(Wd, idxd)
    wq, ws, wS = S.quantize_nvfp4(Wd, idxd, awd)
    big = torch.full((M, 100), 7.0, device="cuda")
    S.splice_gemm_decode_fused(Xd, idxd, axd, wq, ws, awd, wS, out=big[:, :N])
    Y2 = two_call(Xd, idxd, axd, wq, ws, awd, wS, k)
    torch.cuda.synchronize()
    assert torch.equal(big[:, :N], Y2)
    assert torch.all(big[:, N:] == 7.0)
    # K = 0: no channels, Y = 0
    e = torch.zeros(M, 0, dtype=torch.int16, device="cuda")
    w8 = torch.zeros(N, 0, dtype=torch.uint8, device="cuda")
    Y = torch.full((M, N), float("nan"), device="cuda")
    S.splice_gemm_decode_fused(e, None, axd, w8, w8, awd, None, out=Y)
    torch.cuda.synchronize()
    assert torch.equal(Y, torch.zeros_like(Y))


@pytest.mark.parametrize("name", list(synth.QWEN3_8B))
@pytest.mark.parametrize("M", [1, 4])
def test_fused_decode_full_size_sampled(name, M):
    """The decode workload's projections at full size: selection from the
    warm-up on the GPU, then the fused call; 128 sampled output columns
    against the oracle's pipeline, all columns against the two-call form."""
    p = synth.projection(synth.CFG_DECODE, name, M)
    K, N = p["K"], p["N"]
    cols = np.sort(np.random.default_rng(M + 5).choice(N, size=128, replace=False))
    Xw, Xd, Wd = dev(p["X_warm"]), dev(p["X"]), dev(p["W"])
    idx, ax, _ = S.select_channels(Xw, 64)
    aw = S.compute_alpha(Wd, idx)
    wq, ws, wS = S.quantize_nvfp4(Wd, idx, aw)
    Yf = S.splice_gemm_decode_fused(Xd, idx, ax, wq, ws, aw, wS)
    Y2 = two_call(Xd, idx, ax, wq, ws, aw, wS, 64)
    torch.cuda.synchronize()
    # the oracle's own calibration and product on the sampled columns
    oidx, oax, _ = O.select_channels(p["X_warm"], 64)
    assert np.array_equal(host(idx), oidx) and scalar(ax) == np.float32(oax)
    oaw = O.compute_alpha(p["W"], oidx)
    xq, xs, xS = O.quantize_nvfp4(p["X"], oidx, oax)
    wq_o, ws_o, wS_o = O.quantize_nvfp4(p["W"][cols], oidx, oaw)
    Yo = O.splice_gemm(xq, xs, oax, xS, wq_o, ws_o, oaw, wS_o)
    assert_gemm_close(host(Yf)[:, cols], Yo, f"{name} M={M}")
    if same_kernel(M, K):
        assert torch.equal(Yf, Y2), f"{name} M={M}: fused and two-call results differ"
    else:
        assert_gemm_close(host(Yf), host(Y2).astype(np.float64), f"{name} M={M} vs two-call")


def test_fused_decode_in_hip_graph():
    """The fused call captured in a HIP graph: replays with eager work in
    between reproduce the eager result bit for bit."""
    M, N, K, k = 1, 640, 4096, 64
    g = np.random.default_rng(79)
    W = synth.to_bf16(g.normal(0, 0.02, (N, K)))
    Xw = synth.activations(5, 0, 256, K, 2, "student", n_out=16)
    Wd = dev(W)
    idx, ax, _ = S.select_channels(dev(Xw), k)
    aw = S.compute_alpha(Wd, idx)
    wq, ws, wS = S.quantize_nvfp4(Wd, idx, aw)
    xs_in = [dev(synth.activations(5, 0, M, K, 20 + i, "student", n_out=16)) for i in range(3)]
    Xin = torch.empty_like(xs_in[0])
    Y = torch.empty(M, N, device="cuda")

    def call():
        S.splice_gemm_decode_fused(Xin, idx, ax, wq, ws, aw, wS, out=Y)

    eager = []
    for x in xs_in:
        Xin.copy_(x)
        call()
        eager.append(Y.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(2):
        for i, x in enumerate(xs_in):
            Xin.copy_(x)
            Y.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, eager[i]), f"replay {rep} input {i}"
    for i, x in enumerate(xs_in):
        assert torch.equal(eager[i], two_call(x, idx, ax, wq, ws, aw, wS, k))
