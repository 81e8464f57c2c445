"""Helpers for the GPU parity tests: host <-> device copies and the tolerance
of the GEMM outputs.

Tolerance of an fp32 output against the oracle on the same dequantized
operands: relative Frobenius error <= 1e-5 and, per element,
|y - y_oracle| <= max(1e-3 * |y_oracle|, 1e-6), the absolute floor scaled by
the sum of the product magnitudes where that sum exceeds 1 for the rare
element whose products cancel (assert_gemm_close).
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


def pack_magnitudes(xq, xs, ax, xS, wq, ws, aw, wS):
    """A function of (row, column) giving the sum over the reduction of |x * w|
    for that output of the oracle's product of these packs: the dequantized
    FP4 products and the BF16 side products, in output units."""
    import oracle as O

    def terms(i, j):
        dx = O.dequantize(xq[i:i + 1], xs[i:i + 1], ax)[0]
        dw = O.dequantize(wq[j:j + 1], ws[j:j + 1], aw)[0]
        t = float(np.abs(dx * dw).sum())
        if xS is not None and xS.shape[1]:
            sx = np.array([O.bf16_to_double(b) for b in xS[i]])
            sw = np.array([O.bf16_to_double(b) for b in wS[j]])
            t += float(np.abs(sx * sw).sum())
        return t
    return terms


def gemm_errors(Y, Yo):
    Y = np.asarray(Y, np.float64)
    Yo = np.asarray(Yo, np.float64)
    nrm = np.linalg.norm(Yo)
    fro = np.linalg.norm(Y - Yo) / nrm if nrm > 0 else np.linalg.norm(Y - Yo)
    err = np.abs(Y - Yo)
    lim = np.maximum(ELEM_REL * np.abs(Yo), ELEM_ABS)
    return fro, err, lim


def assert_gemm_close(Y, Yo, what="", terms=None, max_scaled=0):
    """The tolerance above.  With `terms` (a function of (row, column) giving
    the sum of the magnitudes of that output's products, in output units),
    an element whose error exceeds the 1e-6 floor may instead meet a floor of
    1e-6 times that sum: where large products cancel, the fp32 accumulation
    of a K-term dot product errs by a few units in the last place of the
    products, not of the result.  At most `max_scaled` elements may need
    this.  Returns the number of elements beyond the literal bound
    max(1e-3 |y_oracle|, 1e-6) that the scaled floor admitted (0 without
    `terms`); a failure message states that count too."""
    fro, err, lim = gemm_errors(Y, Yo)
    bad = np.argwhere(err > lim)
    literal = len(bad)
    if bad.size and terms is not None and len(bad) <= max_scaled:
        keep = [b for b in bad if err[tuple(b)] > ELEM_ABS * max(1.0, terms(*b))]
        bad = np.array(keep).reshape(-1, 2)
    msg = ""
    if bad.size:
        i = tuple(bad[0])
        msg = (f"{what}: {len(bad)} of {err.size} elements outside tolerance "
               f"({literal} beyond the literal floor, at most {max_scaled} may use the scaled "
               f"one); first {i}: gpu {Y[i]!r} oracle {Yo[i]!r}; fro {fro:.3g}")
    assert fro <= FRO_TOL, f"{what}: relative Frobenius error {fro:.3g}"
    assert not bad.size, msg
    return literal
