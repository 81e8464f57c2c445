"""Thin Python binding of libsplice.so (C ABI in include/splice.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library; torch provides device memory and the current HIP
stream.  The library must have been built (python -m fp4_gemm_sparse_amd.build);
loading fails loudly otherwise -- there is no fallback.

bf16 tensors may be torch.bfloat16 or 16-bit integer tensors holding bf16 bit
patterns; codes and scales are torch.uint8; idx is torch.int32; tensor scales
(alpha) are float32 device tensors of one element.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsplice.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "splice.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
SELECT_VARIANCE, SELECT_SECOND_MOMENT = 0, 1
DECODE_MAX_M = 64
FUSED_MAX_M = 4
SEG_MAX = 8

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class SpliceError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({lib().splice_status_string(status).decode()})")


class _Group(ctypes.Structure):
    _fields_ = [("Xq", _vp), ("Xs", _vp), ("alpha_x", _vp), ("X_S", _vp), ("Wq", _vp), ("Ws", _vp),
                ("alpha_w", _vp), ("W_S", _vp), ("M", _i64), ("Y", _vp)]


class _Seg(ctypes.Structure):
    _fields_ = [("Wq", _vp), ("Ws", _vp), ("alpha_w", _vp), ("W_S", _vp), ("N", _i64), ("Y", _vp),
                ("ldy", _i64)]


_SIGS = {
    "splice_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "splice_select_channels": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, ctypes.POINTER(_i64),
                                              _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "splice_select_workspace_size": (_sz, [_i64]),
    "splice_channel_stats": (ctypes.c_int, [_vp, _i64, _i64, _i64, ctypes.POINTER(_i64), _vp, _vp,
                                            _vp, _vp]),
    "splice_select_topk": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, ctypes.c_int, _vp, _vp,
                                          _vp]),
    "splice_compute_alpha": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]),
    "splice_alpha_workspace_size": (_sz, []),
    "splice_quantize_nvfp4": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _vp,
                                             _vp]),
    "splice_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32,
                                   _vp, _i64, _vp, _sz, ctypes.c_int, _vp]),
    "splice_gemm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32,
                                           _vp, _i64, ctypes.c_int, _vp]),
    "nvfp4_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp,
                                  _sz, ctypes.c_int, _vp]),
    "splice_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "splice_multi_workspace_size": (_sz, [_i64, _i64, _i32, ctypes.POINTER(_Seg), _i32]),
    "splice_gemm_plan": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(_i32)]),
    "splice_multi_plan": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_Seg), _i32, ctypes.c_int,
                                         ctypes.POINTER(_i32)]),
    "splice_probe_mfma_f16": (ctypes.c_int, [_i64, _i64, _vp, _vp]),
    "splice_probe_stream_read": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "splice_tim_filter": (ctypes.c_int, [_vp, _i64, _i64, _vp, ctypes.c_float, _i64, _i64, _i64, _vp,
                                         _vp, _vp, _vp, _i64, _i64, _vp]),
    "splice_gemm_decode_fused": (ctypes.c_int, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                                _i64, _i32, _vp, _i64, _vp]),
    "splice_gemm_grouped": (ctypes.c_int, [ctypes.POINTER(_Group), _i32, _i64, _i64, _i32, _vp, _sz,
                                           _vp]),
    "splice_grouped_workspace_size": (_sz, [ctypes.POINTER(_Group), _i32, _i64, _i64, _i32]),
    "splice_gemm_multi": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, ctypes.POINTER(_Seg),
                                         _i32, _vp, _sz, ctypes.c_int, _vp]),
    "splice_gemm_decode_fused_multi": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i32,
                                                      ctypes.POINTER(_Seg), _i32, _vp]),
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp4_gemm_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/splice.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


# ------------------------------------------------------------------ marshalling helpers
def _p(t):
    if t is None:
        return None
    return _vp(t.data_ptr())


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _check(fn, rc):
    if rc != OK:
        raise SpliceError(fn, rc)


def _bf16(t):
    assert t.dtype in (torch.bfloat16, torch.int16, torch.uint16), t.dtype
    assert t.is_cuda
    return t


def _idx(idx, device):
    if idx is None:
        return torch.zeros(0, dtype=torch.int32, device=device)
    assert idx.dtype == torch.int32 and idx.is_cuda
    return idx


# ------------------------------------------------------------------ entry points
@dataclass
class ChannelStats:
    """Running per-channel moments kept on the device."""
    count: int
    mean: torch.Tensor     # float64 [K]
    m2: torch.Tensor       # float64 [K]
    absmax: torch.Tensor   # float32 [K]

    @staticmethod
    def empty(K, device="cuda"):
        return ChannelStats(0, torch.zeros(K, dtype=torch.float64, device=device),
                            torch.zeros(K, dtype=torch.float64, device=device),
                            torch.zeros(K, dtype=torch.float32, device=device))


def select_channels(X, k, stats: ChannelStats | None = None, ldx=None, T=None, out=None):
    """Fold the rows of X (bf16 [T, K]) into `stats` and select the top-k
    channels.  Returns (idx int32 [k] ascending, alpha_x float32 [1], stats).
    out: optional preallocated (idx, alpha_x)."""
    X = _bf16(X)
    K = X.shape[-1]
    if ldx is None:
        ldx = X.stride(0) if X.dim() == 2 else K
    if T is None:
        T = X.shape[0]
    if stats is None:
        stats = ChannelStats.empty(K, X.device)
    if out is None:
        idx = torch.empty(k, dtype=torch.int32, device=X.device)
        alpha = torch.empty(1, dtype=torch.float32, device=X.device)
    else:
        idx, alpha = out
    cnt = _i64(stats.count)
    _check("splice_select_channels",
           lib().splice_select_channels(_p(X), T, K, ldx, k, ctypes.byref(cnt), _p(stats.mean),
                                        _p(stats.m2), _p(stats.absmax), _p(idx), _p(alpha), None, 0,
                                        _stream()))
    stats.count = cnt.value
    return idx, alpha, stats


def channel_stats(X, stats: ChannelStats | None = None, ldx=None, T=None):
    """Fold the rows of X (bf16 [T, K], row stride ldx) into running moments."""
    X = _bf16(X)
    K = X.shape[-1]
    if ldx is None:
        ldx = X.stride(0) if X.dim() == 2 else K
    if T is None:
        T = X.shape[0]
    if stats is None:
        stats = ChannelStats.empty(K, X.device)
    cnt = _i64(stats.count)
    _check("splice_channel_stats",
           lib().splice_channel_stats(_p(X), T, K, ldx, ctypes.byref(cnt), _p(stats.mean),
                                      _p(stats.m2), _p(stats.absmax), _stream()))
    stats.count = cnt.value
    return stats


def select_topk(stats: ChannelStats, k, criterion=SELECT_VARIANCE, out=None):
    """Top-k channels of running moments by variance or second moment.
    Returns (idx int32 [k] ascending, alpha_x float32 [1])."""
    K = stats.m2.numel()
    if out is None:
        idx = torch.empty(k, dtype=torch.int32, device=stats.m2.device)
        alpha = torch.empty(1, dtype=torch.float32, device=stats.m2.device)
    else:
        idx, alpha = out
    _check("splice_select_topk",
           lib().splice_select_topk(_p(stats.mean), _p(stats.m2), _p(stats.absmax), stats.count, K,
                                    k, criterion, _p(idx), _p(alpha), _stream()))
    return idx, alpha


def compute_alpha(A, idx=None, out=None, ws=None):
    A = _bf16(A)
    R, K = A.shape
    idx = _idx(idx, A.device)
    alpha = out if out is not None else torch.empty(1, dtype=torch.float32, device=A.device)
    if ws is None:
        ws = torch.empty(lib().splice_alpha_workspace_size(), dtype=torch.uint8, device=A.device)
    _check("splice_compute_alpha",
           lib().splice_compute_alpha(_p(A), R, K, A.stride(0), _p(idx), idx.numel(), _p(alpha),
                                      _p(ws), ws.numel(), _stream()))
    return alpha


def quantize_nvfp4(A, idx, alpha, out=None):
    """Returns (codes uint8 [R, K/2], scales uint8 [R, K/16], side bf16-bits [R, k])."""
    A = _bf16(A)
    R, K = A.shape
    idx = _idx(idx, A.device)
    k = idx.numel()
    if out is None:
        codes = torch.empty(R, K // 2, dtype=torch.uint8, device=A.device)
        scales = torch.empty(R, K // 16, dtype=torch.uint8, device=A.device)
        side = torch.empty(R, k, dtype=torch.int16, device=A.device)
    else:
        codes, scales, side = out
    _check("splice_quantize_nvfp4",
           lib().splice_quantize_nvfp4(_p(A), R, K, A.stride(0), _p(idx), k, _p(alpha), _p(codes),
                                       _p(scales), _p(side) if k else None, _stream()))
    return codes, scales, side


def workspace_size(M, N, K, k=0):
    return lib().splice_workspace_size(M, N, K, k)


_ws_cache = {}


def workspace(nbytes, device):
    """A zero-filled device workspace of at least nbytes, kept per device and
    reused: the library returns its split counters to zero after every call,
    so calls ordered on one stream can share it (concurrent streams need
    workspaces of their own, passed explicitly).  Grown on demand, which
    allocates: make a first call outside any graph capture."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = t
    return t


def gemm_plan(M, N, K, path=PATH_AUTO):
    """(path taken: 1 decode / 2 prefill, kernel, tile rows, tile columns, K splits)
    of a splice_gemm call of this shape."""
    out = (_i32 * 5)()
    _check("splice_gemm_plan", lib().splice_gemm_plan(M, N, K, path, out))
    return tuple(out)


def multi_plan(M, K, widths, path=PATH_AUTO):
    """The plan of a splice_gemm_multi call with segments of these widths."""
    arr = (_Seg * len(widths))()
    for i, n in enumerate(widths):
        arr[i] = _Seg(None, None, None, None, n, None, n)
    out = (_i32 * 5)()
    _check("splice_multi_plan", lib().splice_multi_plan(M, K, arr, len(widths), path, out))
    return tuple(out)


def splice_gemm(Xq, Xs, alpha_x, X_S, Wq, Ws, alpha_w, W_S, path=PATH_AUTO, out=None, ws=None):
    M, K = Xq.shape[0], Xq.shape[1] * 2
    N = Wq.shape[0]
    k = 0 if X_S is None else X_S.shape[1]
    Y = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=Xq.device)
    need = workspace_size(M, N, K, k)
    if ws is None and need:
        ws = workspace(need, Xq.device)
    _check("splice_gemm",
           lib().splice_gemm(_p(Xq), _p(Xs), _p(alpha_x), _p(X_S) if k else None, _p(Wq), _p(Ws),
                             _p(alpha_w), _p(W_S) if k else None, M, N, K, k, _p(Y), Y.stride(0),
                             _p(ws), 0 if ws is None else ws.numel(), path, _stream()))
    return Y


def splice_gemm_noalloc(Xq, Xs, alpha_x, X_S, Wq, Ws, alpha_w, W_S, path=PATH_AUTO, out=None):
    """splice_gemm with the library's own per-device scratch as workspace:
    nothing is allocated (out must be given for that; calls that overlap on
    one GPU race)."""
    M, K = Xq.shape[0], Xq.shape[1] * 2
    N = Wq.shape[0]
    k = 0 if X_S is None else X_S.shape[1]
    Y = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=Xq.device)
    _check("splice_gemm_noalloc",
           lib().splice_gemm_noalloc(_p(Xq), _p(Xs), _p(alpha_x), _p(X_S) if k else None, _p(Wq), _p(Ws),
                                     _p(alpha_w), _p(W_S) if k else None, M, N, K, k, _p(Y), Y.stride(0),
                                     path, _stream()))
    return Y


def nvfp4_gemm(Xq, Xs, alpha_x, Wq, Ws, alpha_w, path=PATH_AUTO, out=None, ws=None):
    M, K = Xq.shape[0], Xq.shape[1] * 2
    N = Wq.shape[0]
    Y = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=Xq.device)
    need = workspace_size(M, N, K, 0)
    if ws is None and need:
        ws = workspace(need, Xq.device)
    _check("nvfp4_gemm",
           lib().nvfp4_gemm(_p(Xq), _p(Xs), _p(alpha_x), _p(Wq), _p(Ws), _p(alpha_w), M, N, K, _p(Y),
                            Y.stride(0), _p(ws), 0 if ws is None else ws.numel(), path, _stream()))
    return Y


def splice_gemm_decode_fused(X, idx, alpha_x, Wq, Ws, alpha_w, W_S, out=None):
    """Decode SpliceGEMM that quantizes the bf16 activations X [M, K] itself
    (M <= FUSED_MAX_M); idx int32 [k] or None.  Same Y as quantize_nvfp4 then
    splice_gemm."""
    _bf16(X)
    M, K = X.shape
    N = Wq.shape[0]
    k = 0 if idx is None else idx.numel()
    Y = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=X.device)
    _check("splice_gemm_decode_fused",
           lib().splice_gemm_decode_fused(_p(X), X.stride(0), _p(idx) if k else None, _p(alpha_x),
                                          _p(Wq), _p(Ws), _p(alpha_w), _p(W_S) if k else None,
                                          M, N, K, k, _p(Y), Y.stride(0), _stream()))
    return Y


def tim_filter(logp, lengths, log_tau, k1=(1, 100), k2=5, adv=None, out=None):
    """TIM-aware sequence filter.  logp float32 [B, L] (row stride may exceed L),
    lengths int32 [B]; adv float32 [B] or [B, C], masked in place.  Returns
    (keep uint8 [B], G1 int32 [B], G2 int32 [B])."""
    assert logp.dtype == torch.float32 and lengths.dtype == torch.int32
    B = logp.shape[0]
    if out is None:
        keep = torch.empty(B, dtype=torch.uint8, device=logp.device)
        g1 = torch.empty(B, dtype=torch.int32, device=logp.device)
        g2 = torch.empty(B, dtype=torch.int32, device=logp.device)
    else:
        keep, g1, g2 = out
    cols, lda = 0, 0
    if adv is not None:
        assert adv.dtype == torch.float32 and adv.shape[0] == B
        cols = 1 if adv.dim() == 1 else adv.shape[1]
        lda = adv.stride(0) if adv.dim() == 2 else 1
    _check("splice_tim_filter",
           lib().splice_tim_filter(_p(logp), B, logp.stride(0), _p(lengths), float(log_tau), k1[0], k1[1],
                                   k2, _p(keep), _p(g1), _p(g2), _p(adv), cols, lda, _stream()))
    return keep, g1, g2


def probe_mfma_f16(iters, workgroups, sink):
    """Measurement aid: 4 * iters 32x32x16 FP16 MFMAs per wave, 4 waves per
    workgroup (sink float32 [workgroups * 4])."""
    _check("splice_probe_mfma_f16", lib().splice_probe_mfma_f16(iters, workgroups, _p(sink), _stream()))


def probe_stream_read(src, nbytes, workgroups, sink):
    """Measurement aid: a pure read of the first `nbytes` bytes of the device
    tensor src by `workgroups` x 256 threads (sink uint32/int32 [workgroups * 4])."""
    _check("splice_probe_stream_read",
           lib().splice_probe_stream_read(_p(src), nbytes, workgroups, _p(sink), _stream()))


def splice_gemm_multi(Xq, Xs, alpha_x, X_S, weights, path=PATH_AUTO, out=None, ws=None):
    """One launch of the products of one set of activation packs with several
    weight packs.  weights: list of (Wq, Ws, alpha_w, W_S) (W_S None when
    k == 0); out: list of fp32 outputs [M, N_i] or None.  Returns the outputs."""
    M, K = Xq.shape[0], Xq.shape[1] * 2
    k = 0 if X_S is None else X_S.shape[1]
    if out is None:
        out = [torch.empty(M, w[0].shape[0], dtype=torch.float32, device=Xq.device) for w in weights]
    arr = (_Seg * max(len(weights), 1))()
    for i, (w, Y) in enumerate(zip(weights, out)):
        arr[i] = _Seg(_p(w[0]), _p(w[1]), _p(w[2]), _p(w[3]) if k else None, w[0].shape[0], _p(Y),
                      Y.stride(0))
    need = lib().splice_multi_workspace_size(M, K, k, arr, len(weights))
    if ws is None and need:
        ws = workspace(need, Xq.device)
    _check("splice_gemm_multi",
           lib().splice_gemm_multi(_p(Xq), _p(Xs), _p(alpha_x), _p(X_S) if k else None, M, K, k, arr,
                                   len(weights), _p(ws), 0 if ws is None else ws.numel(), path,
                                   _stream()))
    return out


def splice_gemm_decode_fused_multi(X, idx, alpha_x, weights, out=None):
    """splice_gemm_decode_fused over several weight packs in one launch.
    weights: list of (Wq, Ws, alpha_w, W_S); out: list of fp32 [M, N_i] or None."""
    X = _bf16(X)
    M, K = X.shape
    idx = _idx(idx, X.device)
    k = idx.numel()
    if out is None:
        out = [torch.empty(M, w[0].shape[0], dtype=torch.float32, device=X.device) for w in weights]
    arr = (_Seg * max(len(weights), 1))()
    for i, (w, Y) in enumerate(zip(weights, out)):
        arr[i] = _Seg(_p(w[0]), _p(w[1]), _p(w[2]), _p(w[3]) if k else None, w[0].shape[0], _p(Y),
                      Y.stride(0))
    _check("splice_gemm_decode_fused_multi",
           lib().splice_gemm_decode_fused_multi(_p(X), X.stride(0), _p(idx) if k else None, _p(alpha_x),
                                                M, K, k, arr, len(weights), _stream()))
    return out


def splice_gemm_grouped(groups, N, K, k, ws=None):
    """groups: list of dicts with keys Xq, Xs, alpha_x, X_S, Wq, Ws, alpha_w, W_S, Y (device
    tensors; Y fp32 [M, N]).  Each group's M is Xq.shape[0]."""
    arr = (_Group * len(groups))()
    for i, g in enumerate(groups):
        arr[i] = _Group(_p(g["Xq"]), _p(g["Xs"]), _p(g["alpha_x"]), _p(g["X_S"]) if k else None,
                        _p(g["Wq"]), _p(g["Ws"]), _p(g["alpha_w"]), _p(g["W_S"]) if k else None,
                        g["Xq"].shape[0], _p(g["Y"]))
    need = lib().splice_grouped_workspace_size(arr, len(groups), N, K, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _check("splice_gemm_grouped",
           lib().splice_gemm_grouped(arr, len(groups), N, K, k, _p(ws), 0 if ws is None else ws.numel(),
                                     _stream()))
