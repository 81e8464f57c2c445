"""Pins of the oracle's number formats (CPU only).

E2M1 value set: FourSight paper App. 9.3.1 (largest gap 2, largest magnitude 6).
E4M3: OCP E4M3FN, cross-checked against torch.float8_e4m3fn.
The block quantizer is pinned against an exact-rational brute force.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import brute
from fp4_gemm_sparse_amd import synth


def test_e2m1_value_set(oracle_lib):
    o = oracle_lib
    vals = sorted({o.e2m1_decode(c) for c in range(16)})
    assert vals == [-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6]
    pos = [o.e2m1_decode(c) for c in range(8)]
    assert pos == sorted(pos)
    assert max(b - a for a, b in zip(pos, pos[1:])) == 2.0
    assert max(pos) == 6.0
    # sign bit: code 8 is -0
    assert np.signbit(o.e2m1_decode(8)) and not np.signbit(o.e2m1_decode(0))


def test_e2m1_roundtrip(oracle_lib):
    o = oracle_lib
    for c in range(8):
        assert o.e2m1_round(o.e2m1_decode(c)) == c


def test_e2m1_round_exhaustive_bf16(oracle_lib):
    """Every non-negative bf16 value below 8 against the brute-force nearest."""
    o = oracle_lib
    bits = np.arange(0, 0x4100, dtype=np.uint16)   # 0 .. 8.0
    vals = synth.bf16_to_f32(bits).astype(np.float64)
    for v in vals:
        r = Fraction(float(v))
        assert o.e2m1_round(v) == brute.nearest(brute.E2M1, r), v


@pytest.mark.parametrize("r,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                    (3.5, 6), (5.0, 6), (6.0, 7), (7.0, 7), (1e9, 7)])
def test_e2m1_ties_and_saturation(oracle_lib, r, code):
    assert oracle_lib.e2m1_round(r) == code


def test_e4m3_decode_all_bytes(oracle_lib):
    o = oracle_lib
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        got = o.e4m3_decode(b)
        if np.isnan(ref[b]):
            assert np.isnan(got)
        else:
            assert got == ref[b] and np.signbit(got) == np.signbit(ref[b]), b
    assert o.e4m3_decode(0x7E) == 448.0
    assert o.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_roundtrip(oracle_lib):
    o = oracle_lib
    for b in range(0x7F):
        assert o.e4m3_round(o.e4m3_decode(b)) == b


def test_e4m3_round_vs_torch(oracle_lib):
    """RNE agrees with torch's fp32 -> float8_e4m3fn cast on [0, 464]."""
    o = oracle_lib
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.uniform(0, 464, 4000), 2.0 ** g.uniform(-14, 8.8, 4000),
        # every midpoint between neighbours, and its two fp32 neighbours
    ]).astype(np.float32)
    e4 = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((e4[:-1].astype(np.float64) + e4[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    x = x[x <= 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([o.e4m3_round(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(x[i], got[i], ref[i]) for i in bad[:5]]


def test_e4m3_saturates(oracle_lib):
    for v in (448.0, 449.0, 480.0, 1e6, 1e30):
        assert oracle_lib.e4m3_round(v) == 0x7E


def test_alpha_is_correctly_rounded(oracle_lib):
    """alpha = nearest fp32 to amax/2688 (checked in exact rationals)."""
    o = oracle_lib
    bits = np.arange(0x0080, 0x7F80, 97, dtype=np.uint16)   # positive normal bf16 values
    for v in synth.bf16_to_f32(bits):
        a = o.alpha_from_amax(float(v))
        exact = Fraction(float(v)) / 2688
        fa = Fraction(a)
        lo = Fraction(float(np.nextafter(np.float32(a), np.float32(0))))
        hi = Fraction(float(np.nextafter(np.float32(a), np.float32(np.inf))))
        assert abs(fa - exact) <= abs(lo - exact) and abs(fa - exact) <= abs(hi - exact)
    assert o.alpha_from_amax(0.0) == 1.0


def _blocks_quantize_vs_brute(o, xbits, prot_cols, alpha):
    R, K = xbits.shape
    codes, scales, side = o.quantize_nvfp4(xbits, prot_cols, alpha)
    prot = np.zeros(K, bool)
    prot[list(prot_cols)] = True
    for r in range(R):
        for b in range(K // 16):
            sb, nibs = brute.quantize_block(xbits[r, 16 * b:16 * b + 16], prot[16 * b:16 * b + 16],
                                            alpha)
            assert scales[r, b] == sb, (r, b)
            got = []
            for t in range(8):
                byte = codes[r, 8 * b + t]
                got += [byte & 15, byte >> 4]
            assert got == nibs, (r, b, got, nibs)
    assert np.array_equal(side, xbits[:, np.asarray(prot_cols, dtype=np.int64)])


def test_quantize_exhaustive_element_rounding(oracle_lib):
    """All bf16 magnitudes in [0, 6] under a block whose amax is 6 (scale 1,
    alpha 1), both signs: every element decision against the brute force."""
    o = oracle_lib
    mags = np.arange(0, 0x40C1, dtype=np.uint16)          # 0 .. 6.0
    vals = np.concatenate([mags, mags | 0x8000])
    n = (len(vals) + 14) // 15
    vals = np.concatenate([vals, np.zeros(n * 15 - len(vals), np.uint16)]).reshape(n, 15)
    six = synth.bf16_from_f32(np.float32(6.0))
    blocks = np.concatenate([np.full((n, 1), six, np.uint16), vals], axis=1)
    codes, scales, _ = o.quantize_nvfp4(blocks, [], 1.0)
    assert np.all(scales == 0x38)       # e4m3 1.0
    e2 = [brute.nearest(brute.E2M1, Fraction(float(v))) for v in synth.bf16_to_f32(mags)]
    lut = dict(zip(mags.tolist(), e2))
    for r in range(n):
        for t in range(1, 16):
            byte = codes[r, t // 2]
            nib = byte & 15 if t % 2 == 0 else byte >> 4
            b = int(blocks[r, t])
            assert nib == ((8 if b & 0x8000 else 0) | lut[b & 0x7FFF]), (r, t, hex(b))


@pytest.mark.parametrize("alpha", [1.0, 0.37, 2.0 ** -20, 1.0 / 2688, 1e-3 / 3])
def test_quantize_vs_brute_random_blocks(oracle_lib, alpha):
    """Random blocks (normal data, some huge, some tiny, subnormal scales,
    zero blocks, protected lanes) against the exact brute force."""
    o = oracle_lib
    g = np.random.default_rng(11)
    R, K = 6, 128
    x = g.standard_normal((R, K)) * (2.0 ** g.integers(-30, 12, (R, 1)))
    x[0, 16:32] = 0.0                               # zero block
    x[1, 32:48] = -0.0                              # negative zeros
    x[2, :16] *= 1e-6                               # tiny block -> subnormal / zero scale
    x[3, 48:64] = 1e30                              # saturating block
    xbits = synth.to_bf16(x)
    prot = [3, 17, 18, 40, 64, 65, 66, 67, 127]
    _blocks_quantize_vs_brute(o, xbits, prot, alpha)


def test_quantize_all_protected(oracle_lib):
    o = oracle_lib
    x = synth.to_bf16(np.random.default_rng(1).standard_normal((3, 32)))
    codes, scales, side = o.quantize_nvfp4(x, list(range(32)), 0.5)
    assert not codes.any() and not scales.any()
    assert np.array_equal(side, x)


def test_quantize_sign_symmetry(oracle_lib):
    """Q(-x) equals Q(x) with every sign bit flipped."""
    o = oracle_lib
    x = synth.to_bf16(np.random.default_rng(2).standard_normal((4, 64)) * 3)
    prot = [5, 9]
    c1, s1, _ = o.quantize_nvfp4(x, prot, 0.01)
    c2, s2, _ = o.quantize_nvfp4(x ^ np.uint16(0x8000), prot, 0.01)
    assert np.array_equal(s1, s2)
    flip = np.uint8(0x88)
    # protected lanes stay +0 in both
    pmask = np.zeros((4, 64), np.uint8)
    pmask[:, prot] = 8
    pm = (pmask[:, 0::2] | (pmask[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(c2, (c1 ^ flip) ^ pm)


def test_quantize_power_of_two_scaling(oracle_lib):
    """X * 2^p quantized with alpha * 2^p gives the same codes and scales."""
    o = oracle_lib
    xf = np.random.default_rng(3).standard_normal((4, 64))
    x = synth.to_bf16(xf)
    a = o.compute_alpha(x, [7])
    c1, s1, _ = o.quantize_nvfp4(x, [7], a)
    for p in (-5, 3, 17):
        xp = synth.to_bf16(synth.bf16_to_f32(x).astype(np.float64) * 2.0 ** p)
        c2, s2, _ = o.quantize_nvfp4(xp, [7], a * 2.0 ** p)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
