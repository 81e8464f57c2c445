"""Exact-rational brute force used to pin the oracle.

Nothing here shares code with the oracle: values come from the E2M1 value set
the FourSight paper lists (App. 9.3.1) and from torch's own float8_e4m3fn
decoding; every decision is an argmin of exact Fraction distances over the
whole candidate set, ties broken towards the even code.
"""
from fractions import Fraction

import numpy as np
import torch

# E2M1 magnitudes, as the paper lists the finite value set (App. 9.3.1)
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]

# non-negative finite E4M3FN values by byte, decoded by torch
_e4 = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
E4M3 = [Fraction(float(v)) for v in _e4]          # bytes 0x00..0x7E


def nearest(values, r):
    """index of the nearest value to r (exact), ties to the even index."""
    best, bestd = None, None
    for i, v in enumerate(values):
        d = abs(v - r)
        if bestd is None or d < bestd or (d == bestd and i % 2 == 0 and best % 2 == 1):
            best, bestd = i, d
    return best


def bf16_frac(bits):
    u = np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(u))


def quantize_block(xbits, prot, alpha):
    """Brute-force NVFP4 of one 16-element block: returns (scale byte, nibbles)."""
    a = Fraction(float(np.float32(alpha)))
    xs = [Fraction(0) if p else bf16_frac(b) for b, p in zip(xbits, prot)]
    ab = max(abs(x) for x in xs)
    sbyte = nearest(E4M3, ab / (6 * a))
    s = E4M3[sbyte]
    nibs = []
    for b, p, x in zip(xbits, prot, xs):
        neg = (not p) and (int(b) & 0x8000) != 0
        c = 0 if s == 0 else nearest(E2M1, abs(x) / (s * a))
        nibs.append((8 if neg else 0) | c)
    return sbyte, nibs
