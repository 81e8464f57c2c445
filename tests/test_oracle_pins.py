"""Pins of the oracle's GEMM, statistics and selection (CPU only).

Each test checks the oracle against something other than itself: exact
rational arithmetic, a worked example printed in the FourSight paper, the
error bounds the paper proves (App. 9.3, Lemma 2, Lemma 3, Theorem 1), the
special cases k=0 and k=K, and brute-force sorting.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import brute
from fp4_gemm_sparse_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
C_ELEM = 17.0 / 96.0                       # Lemma 2 constant (App. 9.3.2, Eq. 13)


# ------------------------------------------------------------------ worked example
def test_worked_example(oracle_lib):
    o = oracle_lib
    fx = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    blk = synth.to_bf16(np.array([fx["block"]], np.float64))
    for case, prot in (("unprotected", []), ("protect_first", [0])):
        a = o.compute_alpha(blk, prot)
        codes, scales, _ = o.quantize_nvfp4(blk, prot, a)
        phys = o.e4m3_decode(int(scales[0, 0])) * a
        assert phys == pytest.approx(fx[case]["physical_scale"], rel=2.0 ** -22)
        deq = o.dequantize(codes, scales, a)[0]
        np.testing.assert_allclose(deq, fx[case]["dequantized"], rtol=2.0 ** -22, atol=0)


# ------------------------------------------------------------------ GEMM, exact rationals
def _rand_packs(g, R, K):
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = g.integers(0, 0x7F, (R, K // 16), dtype=np.uint8)     # finite, non-negative
    return codes, scales


def _exact_deq(codes, scales):
    e4 = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    R, K2 = codes.shape
    out = [[None] * (2 * K2) for _ in range(R)]
    for r in range(R):
        for j in range(2 * K2):
            b = int(codes[r, j // 2])
            nib = b & 15 if j % 2 == 0 else b >> 4
            v = brute.E2M1[nib & 7] * Fraction(float(e4[scales[r, j // 16]]))
            out[r][j] = -v if nib & 8 else v
    return out


def _fp32_is_nearest(y, exact):
    y = np.float32(y)
    d = abs(Fraction(float(y)) - exact)
    for nb in (np.nextafter(y, np.float32(-np.inf)), np.nextafter(y, np.float32(np.inf))):
        if abs(Fraction(float(nb)) - exact) < d:
            return False
    return True


@pytest.mark.parametrize("M,N,K,k", [(1, 1, 16, 0), (3, 4, 16, 2), (4, 3, 32, 5), (2, 2, 32, 32)])
def test_gemm_exact_rational(oracle_lib, M, N, K, k):
    o = oracle_lib
    g = np.random.default_rng(100 + M * 7 + K + k)
    Xq, Xs = _rand_packs(g, M, K)
    Wq, Ws = _rand_packs(g, N, K)
    X_S = synth.to_bf16(g.standard_normal((M, k)))
    W_S = synth.to_bf16(g.standard_normal((N, k)) * 0.1)
    ax, aw = np.float32(0.013), np.float32(3.7e-4)
    Y = o.splice_gemm(Xq, Xs, ax, X_S, Wq, Ws, aw, W_S)
    xd, wd = _exact_deq(Xq, Xs), _exact_deq(Wq, Ws)
    for m in range(M):
        for n in range(N):
            e = sum(xd[m][j] * wd[n][j] for j in range(K)) * Fraction(float(ax)) * Fraction(float(aw))
            e += sum(brute.bf16_frac(X_S[m, i]) * brute.bf16_frac(W_S[n, i]) for i in range(k))
            assert _fp32_is_nearest(Y[m, n], e), (m, n, Y[m, n], float(e))


def test_nvfp4_is_splice_with_k0(oracle_lib):
    o = oracle_lib
    d = synth.tiny()
    X, W = d["X"][:32], d["W"][:48]
    ax, aw = o.compute_alpha(X, []), o.compute_alpha(W, [])
    Xq, Xs, X_S = o.quantize_nvfp4(X, [], ax)
    Wq, Ws, W_S = o.quantize_nvfp4(W, [], aw)
    a = o.splice_gemm(Xq, Xs, ax, X_S, Wq, Ws, aw, W_S)
    b = o.nvfp4_gemm(Xq, Xs, ax, Wq, Ws, aw)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_all_protected_is_bf16_gemm(oracle_lib):
    o = oracle_lib
    d = synth.tiny()
    X, W = d["X"][:16, :256], d["W"][:24, :256]
    allk = np.arange(256, dtype=np.int32)
    ax, aw = o.compute_alpha(X, allk), o.compute_alpha(W, allk)
    assert ax == 1.0 and aw == 1.0
    Xq, Xs, X_S = o.quantize_nvfp4(X, allk, ax)
    Wq, Ws, W_S = o.quantize_nvfp4(W, allk, aw)
    assert not Xq.any() and not Wq.any() and not Xs.any() and not Ws.any()
    Y = o.splice_gemm(Xq, Xs, ax, X_S, Wq, Ws, aw, W_S)
    Yb, _ = o.bf16_gemm(X, W)
    assert np.array_equal(Y.view(np.uint32), Yb.view(np.uint32))


def test_bf16_gemm_vs_numpy(oracle_lib):
    o = oracle_lib
    d = synth.tiny()
    X, W = d["X"][:8], d["W"][:8]
    _, Y64 = o.bf16_gemm(X, W)
    ref = synth.bf16_to_f32(X).astype(np.float64) @ synth.bf16_to_f32(W).astype(np.float64).T
    np.testing.assert_allclose(Y64, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ error bounds (App. 9.3)
def _quantized_pair(o, X, W, idx):
    ax, aw = o.compute_alpha(X, idx), o.compute_alpha(W, idx)
    xq = o.quantize_nvfp4(X, idx, ax)
    wq = o.quantize_nvfp4(W, idx, aw)
    return ax, aw, xq, wq


def _normal_blocks(o, scales, alpha):
    """mask of blocks whose scale is E4M3-normal and below saturation."""
    s = np.vectorize(o.e4m3_decode)(scales)
    return (s >= 2.0 ** -6) & (scales != 0x7E)


def test_lemma2_element_bound(oracle_lib):
    """|Q(x)-x| <= (17/96) a_b(S) for normal, non-saturating blocks."""
    o = oracle_lib
    d = synth.tiny()
    X = d["X"]
    idx = d["outliers"][:40]
    a = o.compute_alpha(X, idx)
    codes, scales, _ = o.quantize_nvfp4(X, idx, a)
    xr = synth.bf16_to_f32(X).astype(np.float64)
    xr[:, idx] = 0.0
    err = np.abs(o.dequantize(codes, scales, a) - xr)
    ab = np.abs(xr).reshape(X.shape[0], -1, 16).max(axis=2)
    ok = _normal_blocks(o, scales, a)
    # saturating blocks are excluded by the lemma; with alpha from the amax,
    # only the block holding the amax sits at 448, and there v <= 448 exactly
    ok |= (scales == 0x7E)
    bound = (C_ELEM * ab)[:, :, None]
    e = err.reshape(X.shape[0], -1, 16)
    assert ok.mean() > 0.99
    assert np.all(e[ok] <= bound[ok] * (1 + 1e-12))


def test_lemma3_and_theorem1_per_token(oracle_lib):
    """||dx|| <= 4c ||x_R||, ||D||_F <= 4c ||W_R||_F (Lemma 3) and, per token,
    ||y_S - y|| <= sqrt(C) ||W_R||_F ||x_R|| with sqrt(C) = 4c + 4c(1 + 4c),
    C ~= 3.68 (Theorem 1; the proof bounds each sample)."""
    o = oracle_lib
    c = C_ELEM
    sqrtC = 4 * c + 4 * c * (1 + 4 * c)
    assert sqrtC ** 2 == pytest.approx(3.68, abs=0.005)
    d = synth.tiny()
    X, W = d["X"][:64], d["W"][:256]
    for idx in (np.array([], np.int32), d["outliers"], synth.random_channels(0, 0, 1024, 64)):
        ax, aw, (Xq, Xs, X_S), (Wq, Ws, W_S) = _quantized_pair(o, X, W, idx)
        assert _normal_blocks(o, Xs, ax).mean() > 0.99 and _normal_blocks(o, Ws, aw).mean() > 0.99
        xr = synth.bf16_to_f32(X).astype(np.float64)
        wr = synth.bf16_to_f32(W).astype(np.float64)
        xr[:, idx] = 0
        wr[:, idx] = 0
        dx = o.dequantize(Xq, Xs, ax) - xr
        D = o.dequantize(Wq, Ws, aw) - wr
        assert np.all(np.linalg.norm(dx, axis=1) <= 4 * c * np.linalg.norm(xr, axis=1))
        assert np.linalg.norm(D) <= 4 * c * np.linalg.norm(wr)
        Ys = o.splice_gemm(Xq, Xs, ax, X_S, Wq, Ws, aw, W_S).astype(np.float64)
        _, Y = o.bf16_gemm(X, W)
        lhs = np.linalg.norm(Ys - Y, axis=1)
        rhs = sqrtC * np.linalg.norm(wr) * np.linalg.norm(xr, axis=1)
        assert np.all(lhs <= rhs)


def test_exact_split_eq7(oracle_lib):
    """y = W_R x_R + W_S x_S exactly (App. 9.3.1, Eq. 7): with exact
    quantization (every residual value representable), SpliceGEMM returns
    the bf16 product."""
    o = oracle_lib
    g = np.random.default_rng(4)
    # residual entries from the E2M1 set times one common power of two per row,
    # with a 6 in every block so the block scale is exactly 1 (alpha = 2^p/448)
    K = 64
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6])
    X = g.choice(vals, (4, K))
    W = g.choice(vals, (5, K)) * 0.25
    X[:, ::16] = 6.0
    W[:, ::16] = 1.5
    idx = np.array([3, 20, 41], np.int32)
    X[:, idx] = g.standard_normal((4, 3)) * 50
    W[:, idx] = g.standard_normal((5, 3))
    Xb, Wb = synth.to_bf16(X), synth.to_bf16(W)
    ax, aw, (Xq, Xs, X_S), (Wq, Ws, W_S) = _quantized_pair(o, Xb, Wb, idx)
    Ys = o.splice_gemm(Xq, Xs, ax, X_S, Wq, Ws, aw, W_S)
    Yb, _ = o.bf16_gemm(Xb, Wb)
    np.testing.assert_allclose(Ys, Yb, rtol=1e-6, atol=1e-6)


def test_protection_efficacy(oracle_lib):
    """On outlier-heavy inputs, protecting the top-variance channels cuts the
    error against the bf16 product; protecting random channels does not
    (Sec. 6.4, Fig. 13: random selection does not help, variance does)."""
    o = oracle_lib
    d = synth.tiny()
    idx_var, _, _ = o.select_channels(d["X_warm"], 64)
    X, W = d["X"], d["W"]
    _, Yref = o.bf16_gemm(X, W)

    def err(idx):
        ax, aw, (Xq, Xs, X_S), (Wq, Ws, W_S) = _quantized_pair(o, X, W, idx)
        Y = o.splice_gemm(Xq, Xs, ax, X_S, Wq, Ws, aw, W_S).astype(np.float64)
        return np.linalg.norm(Y - Yref) / np.linalg.norm(Yref)

    e0 = err(np.array([], np.int32))
    ev = err(idx_var)
    er = err(synth.random_channels(0, 0, 1024, 64))
    assert ev <= 0.25 * e0, (e0, ev, er)
    assert er >= 0.8 * e0, (e0, ev, er)


# ------------------------------------------------------------------ statistics
def test_stats_exact_rational(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(8)
    T, K = 200, 6                      # several 64-row tiles and a ragged tail
    x = synth.to_bf16(g.standard_normal((T, K)) * 3 + 1.5)
    st = o.stats(x)
    xf = synth.bf16_to_f32(x)
    assert st.count == T
    for j in range(K):
        col = [Fraction(float(v)) for v in xf[:, j]]
        mu = sum(col) / T
        m2 = sum((v - mu) ** 2 for v in col)
        assert st.mean[j] == pytest.approx(float(mu), rel=1e-13, abs=1e-15)
        assert st.m2[j] == pytest.approx(float(m2), rel=1e-12)
        assert st.absmax[j] == np.abs(xf[:, j]).max()


def test_stats_running_merge(oracle_lib):
    """Folding a second batch into running moments matches the moments of the
    concatenation up to rounding; the fold is deterministic."""
    o = oracle_lib
    g = np.random.default_rng(9)
    a = synth.to_bf16(g.standard_normal((130, 5)))
    b = synth.to_bf16(g.standard_normal((77, 5)) * 2 - 1)
    s1 = o.stats(a).update(b)
    s2 = o.stats(np.concatenate([a, b]))
    assert s1.count == 207
    np.testing.assert_allclose(s1.mean, s2.mean, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s1.m2, s2.m2, rtol=1e-12)
    assert np.array_equal(s1.absmax, s2.absmax)
    s3 = o.stats(a).update(b)
    assert np.array_equal(s1.mean.view(np.uint64), s3.mean.view(np.uint64))
    assert np.array_equal(s1.m2.view(np.uint64), s3.m2.view(np.uint64))


def test_stats_row_stride(oracle_lib):
    """ldx subsamples every other row."""
    o = oracle_lib
    x = synth.to_bf16(np.random.default_rng(10).standard_normal((40, 8)))
    st = o.Stats(8).update(x.reshape(-1)[: 39 * 8 + 8].copy(), ldx=16)
    ref = o.stats(x[::2])
    assert st.count == 20
    assert np.array_equal(st.m2.view(np.uint64), ref.m2.view(np.uint64))


# ------------------------------------------------------------------ selection
def test_select_vs_sorted(oracle_lib):
    o = oracle_lib
    g = np.random.default_rng(12)
    m2 = np.round(g.uniform(0, 10, 300), 1)          # many exact ties
    for k in (0, 1, 17, 64, 300):
        want = sorted(sorted(range(300), key=lambda j: (-m2[j], j))[:k])
        assert o.select_topk(m2, k).tolist() == want


def test_select_recovers_planted_outliers(oracle_lib):
    o = oracle_lib
    d = synth.tiny()
    idx, alpha_x, st = o.select_channels(d["X_warm"], 64)
    assert np.array_equal(idx, d["outliers"])
    xr = synth.bf16_to_f32(d["X_warm"]).copy()
    xr[:, idx] = 0
    assert alpha_x == np.float32(np.abs(xr).max()) / np.float32(2688)


# ------------------------------------------------------------------ second-moment selection
def test_second_moments_exact_rational(oracle_lib):
    """m_j = E[x_j^2] formed from the running moments equals the exact mean of
    squares of the bf16 values (the m_j of Prop. 2), over several 64-row tiles
    and two folded batches."""
    o = oracle_lib
    g = np.random.default_rng(21)
    a = synth.to_bf16(g.standard_normal((150, 5)) * 2 + np.array([0, 3, -1, 0.5, 10]))
    b = synth.to_bf16(g.standard_normal((70, 5)) + 1)
    st = o.stats(a).update(b)
    m = o.second_moments(st)
    xf = np.concatenate([synth.bf16_to_f32(a), synth.bf16_to_f32(b)])
    for j in range(5):
        exact = sum(Fraction(float(v)) ** 2 for v in xf[:, j]) / xf.shape[0]
        assert m[j] == pytest.approx(float(exact), rel=1e-12)


def test_second_moments_without_rows(oracle_lib):
    o = oracle_lib
    assert not o.second_moments(o.Stats(7)).any()


def _separated_channels(g, T, K, means):
    """Channels whose standard deviations are spread 1 .. 1 + 0.5 (K - 1) in
    a random order, with the given means."""
    sd = 1.0 + 0.5 * g.permutation(K)
    return synth.to_bf16(g.standard_normal((T, K)) * sd + means)


def test_second_moment_selection_brute_force(oracle_lib):
    """The second-moment top-k equals sorting the exact means of squares
    (ties to the lower index), on channels far from ties."""
    o = oracle_lib
    g = np.random.default_rng(22)
    T, K = 300, 40
    x = _separated_channels(g, T, K, g.uniform(-3, 3, K))
    st = o.stats(x)
    xf = synth.bf16_to_f32(x)
    exact = [sum(Fraction(float(v)) ** 2 for v in xf[:, j]) / T for j in range(K)]
    order = sorted(range(K), key=lambda j: (-exact[j], j))
    for k in (1, 5, 17, 39, 40):
        if k < K:                                  # the case is meaningful: a real gap at the boundary
            assert exact[order[k - 1]] - exact[order[k]] > 1e-6 * exact[order[k - 1]]
        idx, _ = o.select_from_stats(st, k, o.SECOND_MOMENT)
        assert idx.tolist() == sorted(order[:k])


def test_corollary1_gap_condition(oracle_lib):
    """Cor. 1: when the largest squared mean is below the variance gap
    v_(s) - v_(s+1), the top-s variance set is the top-s second-moment set;
    with zero means the two rankings coincide for every s."""
    o = oracle_lib
    g = np.random.default_rng(23)
    T, K, s = 400, 32, 8
    x = _separated_channels(g, T, K, 0.02 * g.standard_normal(K))
    st = o.stats(x)
    v = np.sort(st.m2 / st.count)[::-1]
    assert np.max(st.mean ** 2) < v[s - 1] - v[s]          # the hypothesis holds here
    iv, _ = o.select_from_stats(st, s, o.VARIANCE)
    im, _ = o.select_from_stats(st, s, o.SECOND_MOMENT)
    assert np.array_equal(iv, im)
    # exactly zero means: rows x and -x in pairs, so the second moment is the variance
    half = _separated_channels(g, T // 2, K, 0.0)
    sym = np.empty((T, K), np.uint16)
    sym[0::2] = half
    sym[1::2] = half ^ np.uint16(0x8000)
    st0 = o.stats(sym)
    xf = synth.bf16_to_f32(sym)
    for k in (1, 8, 31):
        want = sorted(sorted(range(K), key=lambda j: (-float(np.sum(xf[:, j].astype(np.float64) ** 2)), j))[:k])
        assert o.select_from_stats(st0, k, o.VARIANCE)[0].tolist() == want
        assert o.select_from_stats(st0, k, o.SECOND_MOMENT)[0].tolist() == want


def test_second_moment_differs_when_the_gap_condition_fails(oracle_lib):
    """A channel with a large mean and almost no spread has the largest
    second moment and the smallest variance: the two criteria disagree, as
    Cor. 1 allows once the squared mean exceeds the variance gap."""
    o = oracle_lib
    g = np.random.default_rng(24)
    T, K = 256, 16
    xr = g.standard_normal((T, K))
    xr[:, 5] = 8.0 + 0.01 * g.standard_normal(T)
    st = o.stats(synth.to_bf16(xr))
    iv, _ = o.select_from_stats(st, 1, o.VARIANCE)
    im, ax_m = o.select_from_stats(st, 1, o.SECOND_MOMENT)
    assert im.tolist() == [5] and iv.tolist() != [5]
    assert int(np.argmin(st.m2)) == 5
    # the frozen scale follows the selected set: channel 5 no longer counts
    assert ax_m == o.alpha_from_absmax(st.absmax, np.array([5], np.int32))
    assert ax_m < o.alpha_from_absmax(st.absmax, iv)
