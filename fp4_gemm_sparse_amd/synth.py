"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random tensors and converts them to bf16 bit
patterns; it holds none of the method's arithmetic and imports neither the
HIP binding nor the oracle.

Workloads stand in for the projections of Qwen3-8B-sized layers (hidden 4096,
MLP 12288, 8 KV heads of 128 -> k/v width 1024) that the FourSight paper
measures on (Sec. 6.3, Fig. 10); the paper's accuracy benchmarks are not used.

Seeds: numpy PCG64 with seed = 1000*cfg + 10*stream + t where
  t = 0 outlier-channel choice, 1 outlier multipliers, 2 warm-up X,
      3 measured X, 4 W, 5 MoE token counts, 6 random-control channels
and `stream` numbers the input stream (one per distinct layer input, or per
expert).  Draws are fp64, rounded to fp32, then to bf16 with
round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

# (K, N) of the seven projections of one Qwen3-8B layer
QWEN3_8B = {
    "q": (4096, 4096),
    "k": (4096, 1024),
    "v": (4096, 1024),
    "o": (4096, 4096),
    "gate": (4096, 12288),
    "up": (4096, 12288),
    "down": (12288, 4096),
}
# which layer input feeds each projection (q/k/v share one, gate/up share one)
INPUT_STREAM = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
PROJ_ID = {name: i for i, name in enumerate(QWEN3_8B)}

CFG_TINY, CFG_DECODE, CFG_PREFILL, CFG_SWEEP, CFG_MOE = 0, 1, 2, 3, 4


def rng(cfg: int, stream: int, t: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg + 10 * stream + t))


def bf16_from_f32(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16(a64) -> np.ndarray:
    return bf16_from_f32(np.asarray(a64, dtype=np.float64).astype(np.float32))


def outlier_channels(cfg: int, stream: int, K: int, n_out: int = 64) -> np.ndarray:
    return np.sort(rng(cfg, stream, 0).choice(K, size=n_out, replace=False)).astype(np.int32)


def activations(cfg: int, stream: int, M: int, K: int, t: int, kind: str,
                n_out: int = 64) -> np.ndarray:
    """X [M,K] as bf16 bits.

    kind "normal":   N(0,1), the outlier channels multiplied by 32 (exact in bf16)
    kind "student":  Student-t with 5 degrees of freedom, the outlier channels
                     multiplied by a per-channel factor drawn from U[20,50]
    """
    ch = outlier_channels(cfg, stream, K, n_out)
    g = rng(cfg, stream, t)
    if kind == "normal":
        x = g.standard_normal((M, K))
        mult = np.full(n_out, 32.0)
    elif kind == "student":
        x = g.standard_t(5.0, (M, K))
        mult = rng(cfg, stream, 1).uniform(20.0, 50.0, n_out)
    else:
        raise ValueError(kind)
    x[:, ch] *= mult
    return to_bf16(x)


def weights(cfg: int, stream: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    return to_bf16(rng(cfg, stream, 4).normal(0.0, std, (N, K)))


def random_channels(cfg: int, stream: int, K: int, k: int) -> np.ndarray:
    return np.sort(rng(cfg, stream, 6).choice(K, size=k, replace=False)).astype(np.int32)


def tiny():
    """M=128, K=N=1024; X ~ N(0,1) with 64 channels x32; W ~ N(0, 0.02);
    512-token warm-up batch.  Returns dict of bf16 bit arrays."""
    K = N = 1024
    return {
        "X_warm": activations(CFG_TINY, 0, 512, K, 2, "normal"),
        "X": activations(CFG_TINY, 0, 128, K, 3, "normal"),
        "W": weights(CFG_TINY, 0, N, K),
        "outliers": outlier_channels(CFG_TINY, 0, K),
    }


SWEEP_KN = (4096, 12288)
SWEEP_MS = (64, 4096)
SWEEP_KS = (0, 64, 128, 256)


def sweep(M: int):
    """Protected-channel sweep inputs: K=4096, N=12288; X ~ N(0,1) with 64
    channels x32; W ~ N(0, 0.02); 512-token warm-up; the 64 random channels of
    the control case."""
    K, N = SWEEP_KN
    return {
        "X_warm": activations(CFG_SWEEP, 0, 512, K, 2, "normal"),
        "X": activations(CFG_SWEEP, 0, M, K, 3, "normal"),
        "W": weights(CFG_SWEEP, 0, N, K),
        "random64": random_channels(CFG_SWEEP, 0, K, 64),
        "K": K,
        "N": N,
    }


def projection(cfg: int, name: str, M: int, kind: str = "student", warm: int = 512):
    """Inputs of one Qwen3-8B-shaped projection: warm-up X, measured X, W."""
    K, N = QWEN3_8B[name]
    s = INPUT_STREAM[name]
    return {
        "X_warm": activations(cfg, s, warm, K, 2, kind),
        "X": activations(cfg, s, M, K, 3, kind),
        "W": weights(cfg, 10 + PROJ_ID[name], N, K),
        "K": K,
        "N": N,
    }


def moe_counts(total: int = 4096, experts: int = 32, cap: int = 512, s: float = 1.2,
               cfg: int = CFG_MOE) -> np.ndarray:
    """Zipf(s)-skewed token counts per expert over a seeded permutation of the
    experts; largest-remainder rounding to `total`; counts above `cap` are
    moved to the lowest-count experts (ties to the lower expert index)."""
    g = rng(cfg, 0, 5)
    w = 1.0 / np.arange(1, experts + 1, dtype=np.float64) ** s
    w = w[g.permutation(experts)]
    share = w / w.sum() * total
    c = np.floor(share).astype(np.int64)
    rem = total - int(c.sum())
    order = sorted(range(experts), key=lambda e: (-(share[e] - c[e]), e))
    for e in order[:rem]:
        c[e] += 1
    excess = int(np.maximum(c - cap, 0).sum())
    c = np.minimum(c, cap)
    while excess > 0:
        e = min(range(experts), key=lambda i: (c[i], i))
        take = min(excess, cap - int(c[e]))
        c[e] += take
        excess -= take
    assert int(c.sum()) == total and c.max() <= cap
    return c


CFG_TIM = 5
TIM_BATCH, TIM_MAX_LEN = 512, 8192        # sequences per step, response limit (8k, Sec. 6.1)


def rollout_logprobs(B: int = TIM_BATCH, L: int = TIM_MAX_LEN, seed: int = 0, tau: float = 1e-4):
    """Per-token training-policy log-probabilities of a rollout batch, float32
    [B, L], and response lengths int32 [B] (tokens past a length are padding).

    Lengths are uniform in [1, L] with a few at the edges (1, 255, 256, 257, L).
    Ordinary tokens have probabilities uniform in [1e-3, 1]; each sequence has
    its own rate of sporadic tail tokens (probabilities in [1e-8, tau]):
    most a low rate (1e-3), one in ten a high one (3e-2, widespread drift),
    one in twenty a run of 3-20 consecutive tail tokens (a degenerate
    stretch), and a few tokens sit exactly at log(tau)."""
    g = np.random.Generator(np.random.PCG64(1000 * CFG_TIM + seed))
    lens = g.integers(1, L + 1, B).astype(np.int32)
    edge = [1, 255, 256, 257, L]
    lens[: min(B, len(edge))] = edge[: min(B, len(edge))]
    lp = np.log(g.uniform(1e-3, 1.0, (B, L))).astype(np.float32)
    rate = np.where(g.random(B) < 0.1, 3e-2, 1e-3)
    tail = g.random((B, L)) < rate[:, None]
    runs = g.random(B) < 0.05
    for i in np.nonzero(runs)[0]:
        n = int(lens[i])
        r = int(g.integers(3, 21))
        s = int(g.integers(0, max(1, n - r + 1)))
        tail[i, s: s + r] = True
    lp[tail] = np.log(g.uniform(1e-8, tau, int(tail.sum()))).astype(np.float32)
    at = g.random((B, L)) < 1e-4
    lp[at] = np.float32(np.log(np.float32(tau)))
    return lp, lens
