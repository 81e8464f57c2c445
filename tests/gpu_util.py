"""Helpers for the GPU parity tests: host <-> device copies and the tolerance
of the GEMM outputs.

Tolerance of an fp32 output against the oracle on the same dequantized
operands: relative Frobenius error <= 1e-5 and, per element,
|y - y_oracle| <= max(1e-3 * |y_oracle|, 1e-6).
"""
import numpy as np
import torch

FRO_TOL = 1e-5
ELEM_REL = 1e-3
ELEM_ABS = 1e-6


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.astype(dtype)


def scalar(t):
    return np.float32(t.item())


def gemm_errors(Y, Yo):
    Y = np.asarray(Y, np.float64)
    Yo = np.asarray(Yo, np.float64)
    nrm = np.linalg.norm(Yo)
    fro = np.linalg.norm(Y - Yo) / nrm if nrm > 0 else np.linalg.norm(Y - Yo)
    err = np.abs(Y - Yo)
    lim = np.maximum(ELEM_REL * np.abs(Yo), ELEM_ABS)
    return fro, err, lim


def assert_gemm_close(Y, Yo, what=""):
    fro, err, lim = gemm_errors(Y, Yo)
    bad = np.argwhere(err > lim)
    msg = ""
    if bad.size:
        i = tuple(bad[0])
        msg = (f"{what}: {len(bad)} of {err.size} elements outside tolerance; first {i}: "
               f"gpu {Y[i]!r} oracle {Yo[i]!r}; fro {fro:.3g}")
    assert fro <= FRO_TOL, f"{what}: relative Frobenius error {fro:.3g}"
    assert not bad.size, msg
