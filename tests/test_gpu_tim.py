"""GPU parity of the TIM-aware sequence filter (splice_tim_filter) against the
oracle: keep flags, both gate counts and the masked advantages bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_gemm_sparse_amd import splice as S
from fp4_gemm_sparse_amd import synth

pytestmark = pytest.mark.gpu

LOG_TAU = np.float32(np.log(np.float32(1e-4)))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def run_both(lp, lens, adv, k1=(1, 100), k2=5, ldl_pad=0):
    B, L = lp.shape
    ko, g1o, g2o, ao = O.tim_filter(lp, lens, LOG_TAU, k1[0], k1[1], k2, adv=adv)
    if ldl_pad:
        big = np.zeros((B, L + ldl_pad), np.float32)
        big[:, :L] = lp
        lpd = torch.from_numpy(big).cuda()[:, :L]
    else:
        lpd = torch.from_numpy(np.ascontiguousarray(lp)).cuda()
    advd = None if adv is None else torch.from_numpy(np.array(adv, np.float32)).cuda()
    keep, g1, g2 = S.tim_filter(lpd, torch.from_numpy(lens).cuda(), LOG_TAU, k1, k2, adv=advd)
    torch.cuda.synchronize()
    assert np.array_equal(keep.cpu().numpy(), ko)
    assert np.array_equal(g1.cpu().numpy(), g1o)
    assert np.array_equal(g2.cpu().numpy(), g2o)
    if adv is not None:
        assert np.array_equal(advd.cpu().numpy().view(np.uint32), ao.view(np.uint32))
    return ko


def test_rollout_batch_full_size():
    """512 responses up to the 8k limit, per-sequence advantages."""
    lp, lens = synth.rollout_logprobs()
    adv = np.random.default_rng(1).standard_normal(len(lens)).astype(np.float32)
    keep = run_both(lp, lens, adv)
    assert 0 < keep.sum() < len(keep)                     # both outcomes occur


@pytest.mark.parametrize("L", [700, 1500])
@pytest.mark.parametrize("pad", [0, 3])
def test_row_strides_and_token_advantages(L, pad):
    """Rows short enough for four waves and long enough for sixteen, with a
    row stride that is (pad 0) or is not (pad 3) a multiple of four floats
    (vector and scalar loads), and per-token advantage rows."""
    lp, lens = synth.rollout_logprobs(B=96, L=L, seed=2 + pad)
    adv = np.random.default_rng(2).standard_normal((96, L)).astype(np.float32)
    run_both(lp, lens, adv, ldl_pad=pad)


@pytest.mark.parametrize("k1,k2", [((1, 4), 3), ((0, 1), 5), ((1, 100), 0), ((7, 3), 1), ((1, 1000), 64)])
def test_other_gate_settings(k1, k2):
    lp, lens = synth.rollout_logprobs(B=64, L=2048, seed=3)
    run_both(lp, lens, None, k1, k2)


def test_edge_lengths():
    """Lengths 0 (dropped: G1 = 0 = K1), 1, around a 256-token chunk, a whole
    row; runs that cross chunk and wave boundaries."""
    L = 4096
    lens = np.array([0, 1, 3, 4, 5, 255, 256, 257, 1023, 1024, 1025, L], np.int32)
    lp = np.full((len(lens), L), np.float32(np.log(0.5)), np.float32)
    lp[:, 250:262] = np.float32(-20.0)                     # a 12-token run across a chunk edge
    lp[:, 1020:1030] = np.float32(-20.0)                   # across a wave segment edge
    lp[-1, ::2] = np.float32(-20.0)
    lp[-1, 3000:3100] = np.float32(-20.0)
    run_both(lp, lens, np.arange(len(lens), dtype=np.float32) - 5)
