"""Hypothesis strategies for adversarial NVFP4 inputs, shared by the CPU
property tests of the oracle and the GPU property tests of the kernels.  No
quantization arithmetic here.

Hypothesis draws a recipe (sizes, which block kinds may appear, the tensor
scale, the protected columns, a seed); numpy expands it into bf16 values, so a
case of thousands of elements costs a handful of draws.  Block kinds:
  - ties: with alpha a power of two and an E4M3 scale s, one element at
    +-6 s alpha (the block's scale is then s) and the others on E2M1 midpoints
    m s alpha, on E2M1 values, at zero, or on the grid s alpha / 8 below the
    block maximum; all exact in bf16, so every midpoint is an exact tie;
  - zero: +0 and -0 only;
  - wide: magnitudes spread over 2^-41 .. 2^32, so the block scales range
    from 0 through the E4M3 subnormals to saturation;
  - saturating: magnitudes above 2688 alpha, where the block scale saturates
    at 448.
No bf16 subnormal is drawn; a protected column may cover whole blocks.
"""
import numpy as np
from hypothesis import strategies as st

from fp4_gemm_sparse_amd import synth

KINDS = ("ties", "zero", "wide", "saturating")
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_value(b):
    e, m = (int(b) >> 3) & 15, int(b) & 7
    return (1 + m / 8) * 2.0 ** (e - 7) if e else m * 2.0 ** -9


def expand(seed, R, nb, alpha_exp, kinds):
    """bf16 bits [R, 16 nb]: every block of a kind drawn from `kinds`."""
    g = np.random.default_rng(seed)
    unit = 2.0 ** alpha_exp
    x = np.empty((R, nb, 16))
    for r in range(R):
        for b in range(nb):
            kind = kinds[g.integers(len(kinds))]
            sign = g.choice([-1.0, 1.0], 16)
            if kind == "ties":
                s = e4m3_value(g.integers(1, 0x7F)) * unit
                pick = g.choice([0, 0, 1, 2, 3], 16)
                v = np.select([pick == 0, pick == 1, pick == 2],
                              [g.choice(MIDPOINTS, 16), g.choice(E2M1_VALUES, 16), np.zeros(16)],
                              g.integers(0, 48, 16) / 8.0) * s * sign
                v[g.integers(16)] = 6.0 * s * g.choice([-1.0, 1.0])
            elif kind == "zero":
                v = np.where(sign < 0, -0.0, 0.0)
            elif kind == "wide":
                v = g.uniform(0.5, 1.0, 16) * 2.0 ** (g.integers(-40, 21) + g.integers(0, 13, 16)) * sign
            else:
                v = g.uniform(0.5, 1.0, 16) * g.uniform(1.01, 1000.0) * 2688.0 * unit * sign
            x[r, b] = v
    return synth.to_bf16(x.reshape(R, 16 * nb))


def alphas(alpha_exp):
    """The tie grid's power of two, or a nearby fp32 value that is not one."""
    return st.sampled_from([1.0, 1.0, 0.75, 1.3, 1.9999]).map(
        lambda f: float(np.float32(2.0 ** alpha_exp * f)))


@st.composite
def protected(draw, nb):
    K = 16 * nb
    prot = set(draw(st.lists(st.integers(0, K - 1), max_size=8)))
    if draw(st.integers(0, 4)) == 0:                      # whole blocks protected
        for b in draw(st.lists(st.integers(0, nb - 1), min_size=1, max_size=2)):
            prot |= set(range(16 * b, 16 * b + 16))
    return sorted(prot)


@st.composite
def operand(draw, R, nb):
    """(bf16 bits [R, 16 nb], alpha)."""
    alpha_exp = draw(st.integers(-30, 30))
    kinds = draw(st.lists(st.sampled_from(KINDS), min_size=1, max_size=4))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    return expand(seed, R, nb, alpha_exp, kinds), draw(alphas(alpha_exp))


@st.composite
def rows(draw, max_blocks=4, max_rows=3):
    """(bf16 bits [R, K], protected columns (sorted, distinct), alpha)."""
    nb = draw(st.integers(1, max_blocks))
    R = draw(st.integers(1, max_rows))
    x, alpha = draw(operand(R, nb))
    return x, draw(protected(nb)), alpha


@st.composite
def gemm_case(draw, max_m=70, max_n=70, min_k128=1, max_k128=3, min_m=1):
    """(X bits [M, K], alpha_x, W bits [N, K], alpha_w, protected columns),
    K a multiple of 128 as the GEMM entry points require."""
    nb = 8 * draw(st.integers(min_k128, max_k128))
    M, N = draw(st.integers(min_m, max_m)), draw(st.integers(1, max_n))
    X, ax = draw(operand(M, nb))
    W, aw = draw(operand(N, nb))
    return X, ax, W, aw, draw(protected(nb))


@st.composite
def channel_moments(draw, max_k_chan=5008):
    """(count, mean fp64 [K], m2 fp64 [K], absmax fp32 [K], k): running
    moments with many exact ties (values drawn from a small pool), zeros,
    subnormal and huge values, and k from 0 to all channels; K a multiple of
    16, as the entry points require."""
    K = draw(st.sampled_from([16, 32, 64, 304, 1024, 4096, max_k_chan]))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    g = np.random.default_rng(seed)
    pool = np.array([0.0, 5e-324, 1e-300, 1.0, 1.0 + 2 ** -52, 2.0, 3.5, 1e10, 1e300])
    kind = draw(st.sampled_from(["pool", "pool", "wide", "integers"]))
    if kind == "pool":
        m2 = g.choice(pool, K)
    elif kind == "wide":
        m2 = np.abs(g.standard_normal(K)) * 10.0 ** g.integers(-300, 300, K)
    else:
        m2 = g.integers(0, 4, K).astype(np.float64)
    count = draw(st.integers(0, 10 ** 6))
    mean = g.standard_normal(K) * 10.0 ** g.integers(-5, 5, K)
    absmax = np.abs(g.standard_normal(K)).astype(np.float32) * np.float32(2.0 ** int(g.integers(-20, 20)))
    k = draw(st.integers(0, min(K, 300)))
    return count, mean, m2, absmax, k


@st.composite
def rollout_batch(draw):
    """(logp float32 [B, L], lengths int32 [B], log_tau, (k1_num, k1_den),
    k2): per-token log-probabilities built from runs of tail tokens (at or
    just below log tau, or far below) and ordinary tokens (at or just above
    log tau, or near 0), so that both gate counts sit near their limits;
    lengths from 0 to L."""
    B = draw(st.integers(1, 300))
    L = draw(st.sampled_from([1, 2, 7, 64, 513, 2048]))
    log_tau = float(np.log(np.float32(draw(st.sampled_from([1e-4, 1e-2, 0.5])))))
    k1 = draw(st.sampled_from([(0, 1), (1, 100), (3, 7), (1, 1), (2, 1000)]))
    k2 = draw(st.integers(0, 40))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    g = np.random.default_rng(seed)
    t = np.float32(log_tau)
    tail = np.array([t, np.nextafter(t, np.float32(-np.inf)), np.float32(-30.0)], np.float32)
    ordinary = np.array([np.nextafter(t, np.float32(np.inf)), np.float32(0.0), np.float32(-1e-3)], np.float32)
    logp = np.empty((B, L), np.float32)
    p_tail = g.uniform(0.0, 0.5)
    for b in range(B):
        j = 0
        while j < L:
            run = int(g.integers(1, 12))
            src = tail if g.random() < p_tail else ordinary
            logp[b, j:j + run] = g.choice(src, min(run, L - j))
            j += run
    lengths = g.integers(0, L + 1, B).astype(np.int32)
    return logp, lengths, log_tau, k1, k2


@st.composite
def token_batches(draw):
    """(K, [(bf16 bits [T, K], row step)...]): two to four batches of token
    rows for running channel moments, each folded through a row stride that
    keeps every row or every second or third one; values normal, tiny, huge,
    constant per channel or zero, so that the Welford updates meet
    cancellation and exact zeros."""
    K = draw(st.sampled_from([16, 48, 256, 1040]))
    nb = draw(st.integers(2, 4))
    out = []
    for _ in range(nb):
        T = draw(st.integers(1, 200))
        step = draw(st.sampled_from([1, 1, 2, 3]))
        kind = draw(st.sampled_from(["normal", "scaled", "constant", "zero", "offset"]))
        g = np.random.default_rng(draw(st.integers(0, 2 ** 32 - 1)))
        if kind == "normal":
            x = g.standard_normal((T, K))
        elif kind == "scaled":
            x = g.standard_normal((T, K)) * 2.0 ** g.integers(-100, 100, K)
        elif kind == "constant":
            x = np.tile(g.standard_normal(K) * 1e3, (T, 1))
        elif kind == "zero":
            x = np.zeros((T, K))
        else:
            x = 1e4 + g.standard_normal((T, K))
        out.append((synth.to_bf16(x), step))
    return K, out


@st.composite
def grouped_case(draw):
    """(N, K, k, [(X bits [M_e, K], alpha_x, W bits [N, K], alpha_w,
    protected columns)...]): 1 to 40 groups sharing N, K and the protected
    count k, each with its own rows (0 to 300), blocks, tensor scales and
    protected set."""
    nb = 8 * draw(st.integers(1, 3))
    K = 16 * nb
    N = draw(st.integers(1, 300))
    k = draw(st.sampled_from([0, 0, 3, 16, 32, 64]))
    groups = []
    for _ in range(draw(st.integers(1, 40))):
        M = draw(st.sampled_from([0, 1, 5, 64, 127, 128, 129, 300]))
        X, ax = draw(operand(M, nb))
        W, aw = draw(operand(N, nb))
        prot = sorted(draw(st.permutations(range(K)))[:k]) if k else []
        groups.append((X, ax, W, aw, prot))
    return N, K, k, groups
