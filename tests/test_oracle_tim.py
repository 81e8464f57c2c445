"""Pins of the oracle's TIM-aware sequence filter (FourSight Sec. 4.1, Eq. 3-4;
settings of Sec. 6.1: tau = 1e-4, K1 = 0.01 x response length, K2 = 5).
CPU only."""
import itertools

import numpy as np
import pytest

import oracle as o

LOG_TAU = np.float32(np.log(np.float32(1e-4)))
TAIL = np.float32(np.log(1e-6))         # pi_train far below tau
BODY = np.float32(np.log(0.5))


def brute(pattern, k1_num=1, k1_den=100, k2=5):
    """Gates written out from their definitions: G1 counts tail tokens, G2 is
    the longest stretch of consecutive tail tokens; the sequence survives
    when G1 < K1 = (k1_num / k1_den) * len and G2 < K2."""
    n = len(pattern)
    g1 = sum(pattern)
    g2 = max((len(list(grp)) for v, grp in itertools.groupby(pattern) if v), default=0)
    keep = (g1 * k1_den < k1_num * n) and (g2 < k2)
    return int(keep), g1, g2


def pattern_rows(patterns, L):
    lp = np.full((len(patterns), L), BODY, np.float32)
    for i, p in enumerate(patterns):
        lp[i, : len(p)] = np.where(np.array(p, bool), TAIL, BODY)
    return lp, np.array([len(p) for p in patterns], np.int32)


@pytest.mark.parametrize("k1,k2", [((1, 100), 5), ((1, 4), 3), ((1, 2), 1), ((0, 1), 9)])
def test_every_tail_pattern_up_to_ten_tokens(k1, k2):
    """All 2047 tail patterns of length 0..10 against the brute-force gates."""
    pats = [p for n in range(11) for p in itertools.product((0, 1), repeat=n)]
    lp, lens = pattern_rows(pats, 10)
    keep, g1, g2, _ = o.tim_filter(lp, lens, LOG_TAU, k1[0], k1[1], k2)
    for i, p in enumerate(pats):
        assert (keep[i], g1[i], g2[i]) == brute(p, k1[0], k1[1], k2), p


def test_tail_threshold_is_inclusive():
    """pi_train <= tau marks a tail token: equality counts, the next float
    above does not."""
    above = np.nextafter(LOG_TAU, np.float32(0))
    lp = np.array([[LOG_TAU, above, LOG_TAU]], np.float32)
    _, g1, g2, _ = o.tim_filter(lp, [3], LOG_TAU)
    assert g1[0] == 2 and g2[0] == 1


def test_padding_is_ignored():
    lp = np.full((2, 40), TAIL, np.float32)
    lp[0, :20] = BODY
    keep, g1, g2, _ = o.tim_filter(lp, [20, 0], LOG_TAU)
    assert g1.tolist() == [0, 0] and g2.tolist() == [0, 0]
    # an empty response: G1 = 0 is not below K1 = 0, so Eq. 3 drops it
    assert keep.tolist() == [1, 0]


def test_cumulative_gate_boundary_is_exact():
    """K1 = 0.01 x 300 = 3: three tail tokens drop the sequence, two keep it
    (compared as 100 * G1 < len, no rounding)."""
    lp = np.full((2, 300), BODY, np.float32)
    lp[0, [10, 100, 200]] = TAIL
    lp[1, [10, 100]] = TAIL
    keep, g1, g2, _ = o.tim_filter(lp, [300, 300], LOG_TAU)
    assert g1.tolist() == [3, 2] and g2.tolist() == [1, 1]
    assert keep.tolist() == [0, 1]


def test_sporadic_jitter_kept_degenerate_run_dropped():
    """Sec. 4.1's two behaviours on a 1000-token response (K1 = 10, K2 = 5):
    nine isolated tail tokens stay; five consecutive ones are dropped by G2
    although G1 = 5 < K1; ten spread ones are dropped by G1."""
    L = 1000
    lp = np.full((4, L), BODY, np.float32)
    lp[0, np.arange(9) * 100 + 7] = TAIL                 # sporadic
    lp[1, 500:505] = TAIL                                # a degenerate stretch
    lp[2, 500:504] = TAIL                                # one short of K2
    lp[3, np.arange(10) * 90 + 3] = TAIL                 # many, none adjacent
    keep, g1, g2, _ = o.tim_filter(lp, [L] * 4, LOG_TAU)
    assert g1.tolist() == [9, 5, 4, 10]
    assert g2.tolist() == [1, 5, 4, 1]
    assert keep.tolist() == [1, 0, 1, 0]


def test_advantages_masked_in_place():
    """Eq. 4: dropped sequences' advantages become +0 (also negative ones);
    kept ones are untouched bit for bit; per-token advantage rows are masked
    whole."""
    g = np.random.default_rng(3)
    B, L = 6, 64
    lp = np.full((B, L), BODY, np.float32)
    lp[[1, 4], 10:16] = TAIL                             # runs of 6 -> dropped
    adv = g.standard_normal(B).astype(np.float32)
    adv[4] = -abs(adv[4])
    keep, _, _, out = o.tim_filter(lp, [L] * B, LOG_TAU, adv=adv)
    assert keep.tolist() == [1, 0, 1, 1, 0, 1]
    assert np.array_equal(out[keep == 1].view(np.uint32), adv[keep == 1].view(np.uint32))
    assert np.array_equal(out[keep == 0].view(np.uint32), np.zeros(2, np.uint32))
    tok = g.standard_normal((B, L)).astype(np.float32)
    _, _, _, out2 = o.tim_filter(lp, [L] * B, LOG_TAU, adv=tok)
    assert not out2[[1, 4]].any() and np.array_equal(out2[keep == 1], tok[keep == 1])
