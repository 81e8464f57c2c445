"""Property tests of the HIP path on adversarial blocks (hypothesis,
derandomized: every run draws the same cases).  The strategies in props.py
build exact E2M1 ties, zero and negative-zero blocks, subnormal and saturated
E4M3 scales, tensor scales from 2^-30 to 2^31 and protected columns that cover
whole blocks.

  - tensor scale, codes, block scales and side columns: bit-exact against the
    oracle;
  - GEMM outputs on both paths: within the worst-case bound of fp32
    summation, |y - y_exact| <= gamma_n * sum |terms| with
    gamma_n = n u / (1 - n u), u = 2^-23 (one unit in the last place per
    rounding, which also covers a truncating adder) and n = K + k + 8
    roundings (K + k sums, the product of the two tensor scales, the final
    fused multiply-add, the partial sums of a split K range).  Every product
    of two decoded FP16 values and of two bf16 values is exact in fp32 and no
    value here is subnormal, so this bound holds for any summation order; the
    per-element relative tolerance of the other parity tests does not, where
    these blocks make products of very different sizes cancel.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from gpu_util import dev, host, scalar
from props import channel_moments, gemm_case, grouped_case, rollout_batch, rows, token_batches

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
U = 2.0 ** -23


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def bf16_values(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


@SETTINGS
@given(rows(max_blocks=40, max_rows=40))
def test_quantize_bit_exact(case):
    A, prot, alpha = case
    idx = np.asarray(prot, np.int32)
    Ad, idxd = dev(A), dev(idx)
    c_o, s_o, side_o = O.quantize_nvfp4(A, idx, np.float32(alpha))
    c_g, s_g, side_g = S.quantize_nvfp4(Ad, idxd, dev(np.array([alpha], np.float32)))
    a_g = S.compute_alpha(Ad, idxd)
    torch.cuda.synchronize()
    assert np.array_equal(host(s_g), s_o)
    assert np.array_equal(host(c_g), c_o)
    if len(prot):
        assert np.array_equal(host(side_g), side_o)
    assert scalar(a_g) == np.float32(O.compute_alpha(A, idx))


def oracle_with_bound(X, ax, W, aw, idx):
    """The oracle's product of these operands and the fp32 summation bound
    of every output (section above)."""
    K = X.shape[1]
    k = len(idx)
    xq, xs, xS = O.quantize_nvfp4(X, idx, ax)
    wq, ws, wS = O.quantize_nvfp4(W, idx, aw)
    Yo = O.splice_gemm(xq, xs, ax, xS, wq, ws, aw, wS).astype(np.float64)
    T = np.abs(O.dequantize(xq, xs, ax)) @ np.abs(O.dequantize(wq, ws, aw)).T
    if k:
        T += np.abs(bf16_values(xS)) @ np.abs(bf16_values(wS)).T
    n = K + k + 8
    return Yo, n * U / (1 - n * U) * T


def check_gemm_bound(case):
    X, ax, W, aw, prot = case
    M, K = X.shape
    N = W.shape[0]
    idx = np.asarray(prot, np.int32)
    k = len(prot)
    ax, aw = np.float32(ax), np.float32(aw)
    xq, xs, xS = O.quantize_nvfp4(X, idx, ax)
    wq, ws, wS = O.quantize_nvfp4(W, idx, aw)
    Yo = O.splice_gemm(xq, xs, ax, xS, wq, ws, aw, wS).astype(np.float64)
    T = np.abs(O.dequantize(xq, xs, ax)) @ np.abs(O.dequantize(wq, ws, aw)).T
    if k:
        T += np.abs(bf16_values(xS)) @ np.abs(bf16_values(wS)).T
    n = K + k + 8
    bound = n * U / (1 - n * U) * T

    Xd, Wd, idxd = dev(X), dev(W), dev(idx)
    axd, awd = dev(np.array([ax], np.float32)), dev(np.array([aw], np.float32))
    gx, gw = S.quantize_nvfp4(Xd, idxd, axd), S.quantize_nvfp4(Wd, idxd, awd)
    torch.cuda.synchronize()
    assert np.array_equal(host(gx[0]), xq) and np.array_equal(host(gx[1]), xs)
    assert np.array_equal(host(gw[0]), wq) and np.array_equal(host(gw[1]), ws)
    paths = [S.PATH_PREFILL] + ([S.PATH_DECODE] if M <= S.DECODE_MAX_M else [])
    for path in paths:
        Y = S.splice_gemm(gx[0], gx[1], axd, gx[2] if k else None, gw[0], gw[1], awd,
                          gw[2] if k else None, path=path)
        err = np.abs(host(Y).astype(np.float64) - Yo)
        bad = np.argwhere(err > bound)
        assert not bad.size, (f"path {path} M={M} N={N} K={K} k={k}: {len(bad)} outside; first "
                              f"{tuple(bad[0])}: err {err[tuple(bad[0])]!r} bound {bound[tuple(bad[0])]!r}")


@SETTINGS
@given(gemm_case())
def test_gemm_within_fp32_summation_bound(case):
    check_gemm_bound(case)


@settings(max_examples=12, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(gemm_case(min_m=5, max_m=20, max_n=80, min_k128=64, max_k128=72))
def test_gemm_bound_with_k_split(case):
    """K = 8192..9216 at 5 to 20 rows and up to 80 columns: both paths split
    the K range over workgroups (the decode path eight ways, the prefill path
    16 or 18)."""
    X, _, W, _, _ = case
    M, K = X.shape
    assert S.gemm_plan(M, W.shape[0], K, S.PATH_DECODE)[4] > 1
    assert S.gemm_plan(M, W.shape[0], K, S.PATH_PREFILL)[4] > 1
    check_gemm_bound(case)


@SETTINGS
@given(channel_moments())
def test_select_topk_bit_exact(case):
    """Top-k by variance and by second moment on moments with many exact
    ties, subnormal and huge values: indices and alpha_x bit-exact against
    the oracle."""
    count, mean, m2, absmax, k = case
    st = O.Stats(len(m2))
    st.count, st.mean, st.m2, st.absmax = count, mean, m2, absmax
    stats = S.ChannelStats(count, dev(mean), dev(m2), dev(absmax))
    for crit, ocrit in ((S.SELECT_VARIANCE, O.VARIANCE), (S.SELECT_SECOND_MOMENT, O.SECOND_MOMENT)):
        idx_o, ax_o = O.select_from_stats(st, k, ocrit)
        idx, ax = S.select_topk(stats, k, crit)
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), idx_o), (crit, k)
        assert scalar(ax) == np.float32(ax_o), (crit, k)


@SETTINGS
@given(rollout_batch())
def test_tim_filter_bit_exact(case):
    """The TIM-aware filter on batches built from runs of tail and ordinary
    tokens, at and next to log tau, with every gate setting drawn: keep, both
    gate counts and the masked advantages bit-exact against the oracle."""
    logp, lengths, log_tau, k1, k2 = case
    B = logp.shape[0]
    adv = np.random.default_rng(B).standard_normal((B, 3)).astype(np.float32)
    ko, g1o, g2o, ao = O.tim_filter(logp, lengths, np.float32(log_tau), k1[0], k1[1], k2, adv=adv)
    advd = dev(adv)
    keep, g1, g2 = S.tim_filter(dev(logp), dev(lengths), np.float32(log_tau), k1, k2, adv=advd)
    torch.cuda.synchronize()
    assert np.array_equal(host(keep), ko)
    assert np.array_equal(host(g1), g1o) and np.array_equal(host(g2), g2o)
    assert np.array_equal(host(advd).view(np.uint32), ao.view(np.uint32))


@SETTINGS
@given(token_batches())
def test_running_channel_stats_bit_exact(case):
    """Running moments folded batch after batch, each through a drawn row
    stride: count, mean, M2 and absmax bit-exact against the oracle's fold
    of the same rows after every batch."""
    K, batches = case
    st_o = O.Stats(K)
    st_g = S.ChannelStats.empty(K)
    for X, step in batches:
        T = (X.shape[0] + step - 1) // step
        st_o.update(np.ascontiguousarray(X[::step]))
        st_g = S.channel_stats(dev(X), st_g, ldx=step * K, T=T)
        torch.cuda.synchronize()
        assert st_g.count == st_o.count
        assert np.array_equal(host(st_g.mean).view(np.uint64), st_o.mean.view(np.uint64))
        assert np.array_equal(host(st_g.m2).view(np.uint64), st_o.m2.view(np.uint64))
        assert np.array_equal(host(st_g.absmax), st_o.absmax)


@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(grouped_case())
def test_grouped_within_fp32_summation_bound(case):
    """The grouped launch over 1 to 40 groups of drawn sizes (empty groups
    included) on adversarial blocks, each with its own tensor scales and
    protected set: every group's output within the fp32 summation bound of
    the oracle's product."""
    N, K, k, groups = case
    dgroups, refs = [], []
    for X, ax, W, aw, prot in groups:
        M = X.shape[0]
        idx = np.asarray(prot, np.int32)
        ax32, aw32 = np.float32(ax), np.float32(aw)
        axd, awd = dev(np.array([ax32], np.float32)), dev(np.array([aw32], np.float32))
        if M:
            gx = S.quantize_nvfp4(dev(X), dev(idx), axd)
            refs.append(oracle_with_bound(X, ax32, W, aw32, idx))
        else:
            gx = (torch.zeros(0, K // 2, dtype=torch.uint8, device="cuda"),
                  torch.zeros(0, K // 16, dtype=torch.uint8, device="cuda"),
                  torch.zeros(0, max(k, 1), dtype=torch.int16, device="cuda"))
            refs.append(None)
        gw = S.quantize_nvfp4(dev(W), dev(idx), awd)
        dgroups.append(dict(Xq=gx[0], Xs=gx[1], alpha_x=axd, X_S=gx[2], Wq=gw[0], Ws=gw[1], alpha_w=awd,
                            W_S=gw[2], Y=torch.full((M, N), float("nan"), device="cuda")))
    S.splice_gemm_grouped(dgroups, N, K, k)
    torch.cuda.synchronize()
    for e, (g, ref) in enumerate(zip(dgroups, refs)):
        if ref is None:
            continue
        Yo, bound = ref
        err = np.abs(host(g["Y"]).astype(np.float64) - Yo)
        bad = np.argwhere(~(err <= bound))
        assert not bad.size, f"group {e} of {len(groups)}: M={g['Y'].shape[0]} N={N} K={K} k={k}: {len(bad)} outside"
