"""Property tests of the oracle's NVFP4 quantization (hypothesis, derandomized
so that every run draws the same cases) on adversarial blocks: exact ties on
E2M1 midpoints, zero and negative-zero blocks, subnormal E4M3 scales, a frozen
scale that saturates, protected lanes and whole protected blocks (the
strategies in props.py).  The reference is the exact-rational brute force of
brute.py, which shares nothing with the oracle."""
import numpy as np
from hypothesis import HealthCheck, given, settings

import brute
from props import channel_moments, rows

SETTINGS = settings(max_examples=250, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


@SETTINGS
@given(rows())
def test_quantize_matches_brute_force(oracle_lib, case):
    xbits, prot, alpha = case
    R, K = xbits.shape
    codes, scales, side = oracle_lib.quantize_nvfp4(xbits, prot, alpha)
    pm = np.zeros(K, bool)
    pm[prot] = True
    for r in range(R):
        for b in range(K // 16):
            sb, nibs = brute.quantize_block(xbits[r, 16 * b:16 * b + 16], pm[16 * b:16 * b + 16], alpha)
            assert scales[r, b] == sb, (r, b)
            got = [v for byte in codes[r, 8 * b:8 * b + 8] for v in (byte & 15, byte >> 4)]
            assert got == nibs, (r, b, got, nibs)
    assert np.array_equal(side, xbits[:, np.asarray(prot, dtype=np.int64)])


@SETTINGS
@given(rows())
def test_quantize_sign_symmetry(oracle_lib, case):
    """Q(-x) is Q(x) with the sign bit of every unprotected code flipped;
    scales and side columns follow x."""
    xbits, prot, alpha = case
    c1, s1, side1 = oracle_lib.quantize_nvfp4(xbits, prot, alpha)
    c2, s2, side2 = oracle_lib.quantize_nvfp4(xbits ^ np.uint16(0x8000), prot, alpha)
    assert np.array_equal(s1, s2)
    assert np.array_equal(side2, side1 ^ np.uint16(0x8000))
    n1 = np.stack([c1 & 15, c1 >> 4], -1).reshape(c1.shape[0], -1)
    n2 = np.stack([c2 & 15, c2 >> 4], -1).reshape(c2.shape[0], -1)
    pm = np.zeros(n1.shape[1], bool)
    pm[prot] = True
    # unprotected lanes flip their sign bit, protected lanes stay +0
    assert np.array_equal(n2[:, ~pm], n1[:, ~pm] ^ 8)
    assert not n1[:, pm].any() and not n2[:, pm].any()


def brute_topk(values, k):
    """The k largest values, ties to the lower index, as ascending indices."""
    order = sorted(range(len(values)), key=lambda j: (-values[j], j))
    return np.sort(np.asarray(order[:k], dtype=np.int64))


@settings(max_examples=150, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(channel_moments())
def test_select_topk_matches_sort(oracle_lib, case):
    """The oracle's top-k against a plain sort, on values with many exact
    ties: the set is the k largest and ties go to the lower index."""
    _, _, m2, _, k = case
    assert np.array_equal(oracle_lib.select_topk(m2, k), brute_topk(m2, k))
