"""fp64 CPU oracle for SpliceGEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the cpu_baseline leg of
bench.py may import this package.  The product path (fp4_gemm_sparse_amd)
never imports it, and it imports nothing from the product path.

Thin ctypes marshalling over oracle/oracle.c (host memory, numpy arrays).
Every numerical step lives in the C file, which cites the passages of the
FourSight paper (arXiv 2611.04887v1) it follows.

bf16 tensors are passed as numpy uint16 arrays holding the bit patterns.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle.build import build
            build()
        L = ctypes.CDLL(_LIB_PATH)
        sig = {
            "oracle_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "oracle_e2m1_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_e2m1_round": (ctypes.c_uint8, [ctypes.c_double]),
            "oracle_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_e4m3_round": (ctypes.c_uint8, [ctypes.c_double]),
            "oracle_alpha_from_amax": (ctypes.c_float, [ctypes.c_float]),
            "oracle_compute_alpha": (ctypes.c_int, [_u16p, _i64, _i64, _i64, _i32p, _i32, _f32p]),
            "oracle_alpha_from_absmax": (ctypes.c_int, [_f32p, _i64, _i32p, _i32, _f32p]),
            "oracle_quantize_nvfp4": (ctypes.c_int, [_u16p, _i64, _i64, _i64, _i32p, _i32,
                                                     ctypes.c_float, _u8p, _u8p, _u16p]),
            "oracle_dequantize": (ctypes.c_int, [_u8p, _u8p, ctypes.c_float, _i64, _i64, _f64p]),
            "oracle_splice_gemm": (ctypes.c_int, [_u8p, _u8p, ctypes.c_float, _u16p,
                                                  _u8p, _u8p, ctypes.c_float, _u16p,
                                                  _i64, _i64, _i64, _i32, _f32p, _i64]),
            "oracle_nvfp4_gemm": (ctypes.c_int, [_u8p, _u8p, ctypes.c_float,
                                                 _u8p, _u8p, ctypes.c_float,
                                                 _i64, _i64, _i64, _f32p, _i64]),
            "oracle_bf16_gemm": (ctypes.c_int, [_u16p, _u16p, _i64, _i64, _i64, _i64, _i64,
                                                _f32p, _f64p]),
            "oracle_stats": (ctypes.c_int, [_u16p, _i64, _i64, _i64, _i64p, _f64p, _f64p, _f32p]),
            "oracle_select_topk": (ctypes.c_int, [_f64p, _i64, _i32, _i32p]),
            "oracle_second_moments": (ctypes.c_int, [_f64p, _f64p, _i64, _i64, _f64p]),
            "oracle_select_channels": (ctypes.c_int, [_u16p, _i64, _i64, _i64, _i32, _i64p,
                                                      _f64p, _f64p, _f32p, _i32p, _f32p]),
            "oracle_num_threads": (ctypes.c_int, []),
            "oracle_tim_filter": (ctypes.c_int, [_f32p, _i64, _i64, _i32p, ctypes.c_float, _i64,
                                                 _i64, _i64, _u8p, _i32p, _i32p, _f32p, _i64,
                                                 _i64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


# ---------------------------------------------------------------- codecs
def bf16_to_double(b):
    return lib().oracle_bf16_to_double(int(b))


def e2m1_decode(nib):
    return lib().oracle_e2m1_decode(int(nib))


def e2m1_round(r):
    return int(lib().oracle_e2m1_round(float(r)))


def e4m3_decode(b):
    return lib().oracle_e4m3_decode(int(b))


def e4m3_round(v):
    return int(lib().oracle_e4m3_round(float(v)))


def alpha_from_amax(amax):
    return float(np.float32(lib().oracle_alpha_from_amax(float(amax))))


# ---------------------------------------------------------------- ops
def _idx(idx):
    idx = _c(np.asarray(idx, dtype=np.int32).reshape(-1), np.int32)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)[:0]
    return idx


def compute_alpha(A, idx):
    A = _c(A, np.uint16)
    R, K = A.shape
    idx = _idx(idx)
    out = ctypes.c_float()
    buf = idx if idx.size else np.zeros(1, np.int32)
    _check(lib().oracle_compute_alpha(_p(A, _u16p), R, K, K, _p(buf, _i32p), idx.size,
                                      ctypes.byref(out)), "compute_alpha")
    return float(np.float32(out.value))


def alpha_from_absmax(absmax, idx):
    absmax = _c(absmax, np.float32)
    idx = _idx(idx)
    buf = idx if idx.size else np.zeros(1, np.int32)
    out = ctypes.c_float()
    _check(lib().oracle_alpha_from_absmax(_p(absmax, _f32p), absmax.size, _p(buf, _i32p),
                                          idx.size, ctypes.byref(out)), "alpha_from_absmax")
    return float(np.float32(out.value))


def quantize_nvfp4(A, idx, alpha):
    """Returns (codes u8 [R,K/2], scales u8 [R,K/16], side u16 [R,k])."""
    A = _c(A, np.uint16)
    R, K = A.shape
    idx = _idx(idx)
    k = idx.size
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, max(K // 16, 0)), np.uint8)
    side = np.zeros((R, k), np.uint16)
    buf = idx if k else np.zeros(1, np.int32)
    sbuf = side if side.size else np.zeros(1, np.uint16)
    _check(lib().oracle_quantize_nvfp4(_p(A, _u16p), R, K, K, _p(buf, _i32p), k,
                                       ctypes.c_float(alpha), _p(codes, _u8p), _p(scales, _u8p),
                                       _p(sbuf, _u16p)), "quantize_nvfp4")
    return codes, scales, side


def dequantize(codes, scales, alpha):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    R, K2 = codes.shape
    out = np.zeros((R, 2 * K2), np.float64)
    _check(lib().oracle_dequantize(_p(codes, _u8p), _p(scales, _u8p), ctypes.c_float(alpha),
                                   R, 2 * K2, _p(out, _f64p)), "dequantize")
    return out


def splice_gemm(Xq, Xs, alpha_x, X_S, Wq, Ws, alpha_w, W_S):
    Xq, Xs, Wq, Ws = (_c(a, np.uint8) for a in (Xq, Xs, Wq, Ws))
    M, K2 = Xq.shape
    N = Wq.shape[0]
    K = 2 * K2
    X_S = _c(X_S, np.uint16).reshape(M, -1) if X_S is not None else np.zeros((M, 0), np.uint16)
    W_S = _c(W_S, np.uint16).reshape(N, -1) if W_S is not None else np.zeros((N, 0), np.uint16)
    k = X_S.shape[1]
    assert W_S.shape[1] == k
    Y = np.zeros((M, N), np.float32)
    xs = X_S if X_S.size else np.zeros(1, np.uint16)
    ws = W_S if W_S.size else np.zeros(1, np.uint16)
    _check(lib().oracle_splice_gemm(_p(Xq, _u8p), _p(Xs, _u8p), ctypes.c_float(alpha_x),
                                    _p(xs, _u16p), _p(Wq, _u8p), _p(Ws, _u8p),
                                    ctypes.c_float(alpha_w), _p(ws, _u16p), M, N, K, k,
                                    _p(Y, _f32p), N), "splice_gemm")
    return Y


def nvfp4_gemm(Xq, Xs, alpha_x, Wq, Ws, alpha_w):
    Xq, Xs, Wq, Ws = (_c(a, np.uint8) for a in (Xq, Xs, Wq, Ws))
    M, K2 = Xq.shape
    N = Wq.shape[0]
    Y = np.zeros((M, N), np.float32)
    _check(lib().oracle_nvfp4_gemm(_p(Xq, _u8p), _p(Xs, _u8p), ctypes.c_float(alpha_x),
                                   _p(Wq, _u8p), _p(Ws, _u8p), ctypes.c_float(alpha_w),
                                   M, N, 2 * K2, _p(Y, _f32p), N), "nvfp4_gemm")
    return Y


def bf16_gemm(X, W):
    """Returns (Y fp32, Y fp64) of the unquantized bf16 product X W^T."""
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    M, K = X.shape
    N = W.shape[0]
    Y = np.zeros((M, N), np.float32)
    Y64 = np.zeros((M, N), np.float64)
    _check(lib().oracle_bf16_gemm(_p(X, _u16p), _p(W, _u16p), M, N, K, K, K, _p(Y, _f32p),
                                  _p(Y64, _f64p)), "bf16_gemm")
    return Y, Y64


class Stats:
    """Running per-channel moments (count, mean, M2, absmax)."""

    def __init__(self, K):
        self.K = K
        self.count = 0
        self.mean = np.zeros(K, np.float64)
        self.m2 = np.zeros(K, np.float64)
        self.absmax = np.zeros(K, np.float32)

    def update(self, X, ldx=None):
        X = _c(X, np.uint16)
        if ldx is None:
            T, K = X.shape
            ldx = K
        else:
            K = self.K
            T = (X.size - K) // ldx + 1 if X.size else 0
        assert K == self.K
        cnt = ctypes.c_int64(self.count)
        _check(lib().oracle_stats(_p(X, _u16p), T, K, ldx, ctypes.byref(cnt),
                                  _p(self.mean, _f64p), _p(self.m2, _f64p),
                                  _p(self.absmax, _f32p)), "stats")
        self.count = cnt.value
        return self


def stats(X):
    return Stats(np.asarray(X).shape[1]).update(X)


def select_topk(m2, k):
    m2 = _c(m2, np.float64)
    idx = np.zeros(max(k, 1), np.int32)
    _check(lib().oracle_select_topk(_p(m2, _f64p), m2.size, k, _p(idx, _i32p)), "select_topk")
    return idx[:k].copy()


VARIANCE, SECOND_MOMENT = "variance", "second_moment"


def second_moments(st):
    """E[x^2] per channel from running moments: m2/n + mean^2."""
    out = np.zeros(st.K, np.float64)
    mean = _c(st.mean, np.float64)
    m2 = _c(st.m2, np.float64)
    _check(lib().oracle_second_moments(_p(mean, _f64p), _p(m2, _f64p), st.count, st.K,
                                       _p(out, _f64p)), "second_moments")
    return out


def select_from_stats(st, k, criterion=VARIANCE):
    """Top-k channels of running moments by variance (M2) or by second
    moment, and the frozen activation scale."""
    if criterion == VARIANCE:
        idx = select_topk(st.m2, k)
    elif criterion == SECOND_MOMENT:
        idx = select_topk(second_moments(st), k)
    else:
        raise ValueError(criterion)
    return idx, alpha_from_absmax(st.absmax, idx)


def select_channels(X, k, criterion=VARIANCE):
    """Calibration on a warm-up batch: returns (idx, alpha_x, Stats)."""
    st = stats(X)
    idx, ax = select_from_stats(st, k, criterion)
    return idx, ax, st


def tim_filter(logp, lengths, log_tau, k1_num=1, k1_den=100, k2=5, adv=None):
    """TIM-aware sequence filter over per-token log-probabilities logp
    float32 [B, L] (tokens t >= lengths[i] are padding).  Returns
    (keep u8 [B], G1 int32 [B], G2 int32 [B], masked copy of adv or None);
    adv is float32 [B] or [B, C]."""
    logp = _c(logp, np.float32)
    B, L = logp.shape
    lengths = _c(lengths, np.int32)
    keep = np.zeros(max(B, 1), np.uint8)
    g1 = np.zeros(max(B, 1), np.int32)
    g2 = np.zeros(max(B, 1), np.int32)
    out = None
    cols = 0
    if adv is not None:
        out = np.array(adv, np.float32, copy=True).reshape(B, -1)
        cols = out.shape[1]
    lp = logp if logp.size else np.zeros(1, np.float32)
    ln = lengths if lengths.size else np.zeros(1, np.int32)
    ob = out if (out is not None and out.size) else np.zeros(1, np.float32)
    _check(lib().oracle_tim_filter(_p(lp, _f32p), B, L, _p(ln, _i32p), np.float32(log_tau), k1_num,
                                   k1_den, k2, _p(keep, _u8p), _p(g1, _i32p), _p(g2, _i32p),
                                   _p(ob, _f32p), cols, cols), "tim_filter")
    if out is not None:
        out = out.reshape(np.shape(adv))
    return keep[:B].copy(), g1[:B].copy(), g2[:B].copy(), out


def num_threads():
    return int(lib().oracle_num_threads())
