"""C ABI of libsplice.so on the CPU: the library loads, exports every function
include/splice.h declares, and rejects bad arguments on the host before it
touches a GPU (no compute call is made here)."""
import ctypes

import pytest

from fp4_gemm_sparse_amd import splice

FAKE = 0x100000          # a 16-byte aligned non-null address that is never dereferenced


@pytest.fixture(scope="module")
def L():
    return splice.lib()


def test_exports_every_declared_symbol(L):
    names = splice.header_functions()
    assert {"splice_select_channels", "splice_quantize_nvfp4", "splice_gemm", "nvfp4_gemm",
            "splice_compute_alpha", "splice_gemm_grouped", "splice_workspace_size",
            "splice_gemm_multi", "splice_gemm_decode_fused_multi"} <= set(names)
    for n in names:
        assert getattr(L, n) is not None


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(L.splice_status_string(code), bytes)


def gemm(L, M=64, N=64, K=256, k=8, path=0, ws=None, wsb=0, **over):
    args = dict(Xq=FAKE, Xs=FAKE, ax=FAKE, XS=FAKE, Wq=FAKE, Ws=FAKE, aw=FAKE, WS=FAKE, Y=FAKE,
                ldy=N)
    args.update(over)
    return L.splice_gemm(args["Xq"], args["Xs"], args["ax"], args["XS"], args["Wq"], args["Ws"],
                         args["aw"], args["WS"], M, N, K, k, args["Y"], args["ldy"], ws, wsb, path,
                         None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=100), splice.ERR_INVALID_ARG),            # K % 16
    (dict(K=256, k=257), splice.ERR_INVALID_ARG),     # k > K
    (dict(k=-1), splice.ERR_INVALID_ARG),
    (dict(M=-1), splice.ERR_INVALID_ARG),
    (dict(K=144), splice.ERR_UNSUPPORTED),            # GEMM kernels need K % 128
    (dict(K=131072), splice.ERR_UNSUPPORTED),         # beyond the largest K
    (dict(path=7), splice.ERR_INVALID_ARG),
    (dict(M=65, path=splice.PATH_DECODE), splice.ERR_INVALID_ARG),
    (dict(Y=None), splice.ERR_INVALID_ARG),
    (dict(ax=None), splice.ERR_INVALID_ARG),
    (dict(Xq=None), splice.ERR_INVALID_ARG),
    (dict(XS=None), splice.ERR_INVALID_ARG),
    (dict(Xq=FAKE + 4), splice.ERR_INVALID_ARG),      # misaligned codes
    (dict(Ws=FAKE + 8), splice.ERR_INVALID_ARG),      # scales are loaded as 16-byte vectors
    (dict(Xs=FAKE + 8), splice.ERR_INVALID_ARG),
    (dict(ldy=10), splice.ERR_INVALID_ARG),
    (dict(M=0), splice.OK),                           # no-op
    (dict(N=0), splice.OK),
])
def test_gemm_argument_errors(L, kw, code):
    assert gemm(L, **kw) == code


def test_gemm_workspace_size(L):
    # either path splits K (and needs a workspace) only where its tiles or
    # column groups alone leave CUs idle, and the size covers a call forced
    # onto either path
    for M, N, K, k in ((8192, 4096, 4096, 64), (4096, 12288, 4096, 64), (0, 1024, 4096, 64)):
        assert L.splice_workspace_size(M, N, K, k) == 0
    for M, N, K in ((1, 1024, 4096), (64, 4096, 4096), (65, 4096, 4096), (128, 1024, 4096),
                    (512, 1024, 4096), (200, 300, 12288)):
        assert 0 < L.splice_workspace_size(M, N, K, 64) <= 17 << 20
    assert L.splice_workspace_size(8, 1024, 512, 0) == 0        # too few K steps to split


def test_gemm_missing_workspace(L):
    need = L.splice_workspace_size(128, 1024, 4096, 64)
    assert gemm(L, M=128, N=1024, K=4096, k=64) == splice.ERR_WORKSPACE
    assert gemm(L, M=128, N=1024, K=4096, k=64, ws=FAKE, wsb=need - 1) == splice.ERR_WORKSPACE
    assert gemm(L, M=128, N=1024, K=4096, k=64, ws=FAKE + 8, wsb=need) == splice.ERR_WORKSPACE
    # a decode-path call whose K range is split (M = 64, N = 1024)
    assert splice.gemm_plan(64, 1024, 4096, splice.PATH_DECODE)[4] > 1
    assert gemm(L, M=64, N=1024, K=4096, k=64, path=splice.PATH_DECODE) == splice.ERR_WORKSPACE


def test_multi_workspace_size(L):
    S = splice._Seg
    segs = (S * 3)(S(FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 4096), S(FAKE, FAKE, FAKE, FAKE, 1000, FAKE, 1000),
                   S(FAKE, FAKE, FAKE, FAKE, 1000, FAKE, 1000))
    # 128-column tiles are counted per segment: 32 + 8 + 8, more than the 48 of one 6000-wide call
    multi = L.splice_multi_workspace_size(128, 4096, 64, segs, 3)
    assert multi >= L.splice_workspace_size(128, 6000, 4096, 64) > 0
    assert L.splice_multi_workspace_size(8192, 4096, 64, segs, 3) == 0


def test_noalloc_argument_errors(L):
    f = L.splice_gemm_noalloc
    args = lambda **o: [o.get(n, FAKE) for n in ("Xq", "Xs", "ax", "XS", "Wq", "Ws", "aw", "WS")]
    assert f(*args(), 4, 64, 100, 8, FAKE, 64, 0, None) == splice.ERR_INVALID_ARG      # K % 16
    assert f(*args(), 4, 64, 144, 8, FAKE, 64, 0, None) == splice.ERR_UNSUPPORTED      # K % 128
    assert f(*args(Ws=FAKE + 8), 4, 64, 256, 8, FAKE, 64, 0, None) == splice.ERR_INVALID_ARG
    assert f(*args(), 65, 64, 256, 8, FAKE, 64, splice.PATH_DECODE, None) == splice.ERR_INVALID_ARG
    assert f(*args(), 0, 64, 256, 8, FAKE, 64, 0, None) == splice.OK                   # no-op
    # every shape's workspace fits the library's array (16 MiB + 1 KB)
    for M, N, K in ((65, 64, 17408), (128, 1024, 4096), (100, 128, 65536), (127, 127, 12288)):
        assert L.splice_workspace_size(M, N, K, 0) <= 16 * 1024 * 1024 + 1024


def test_nvfp4_argument_errors(L):
    assert L.nvfp4_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, 4, None, 0, 0, None) \
        == splice.ERR_INVALID_ARG
    assert L.nvfp4_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 128, FAKE, 4, None, 0, 0, None) \
        == splice.OK


def test_quantize_argument_errors(L):
    q = L.splice_quantize_nvfp4
    assert q(FAKE, 4, 100, 100, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert q(FAKE, 4, 64, 32, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # lda < K
    assert q(FAKE, 4, 64, 64, None, 1, FAKE, FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # idx
    assert q(FAKE, 4, 64, 64, FAKE, 1, FAKE, FAKE, FAKE, None, None) == splice.ERR_INVALID_ARG   # side
    assert q(FAKE, 4, 64, 64, FAKE, 0, None, FAKE, FAKE, None, None) == splice.ERR_INVALID_ARG   # alpha
    assert q(FAKE, 4, 64, 68, FAKE, 0, FAKE, FAKE, FAKE, None, None) == splice.ERR_UNSUPPORTED   # lda % 8
    assert q(FAKE + 2, 4, 64, 64, FAKE, 0, FAKE, FAKE, FAKE, None, None) == splice.ERR_UNSUPPORTED
    assert q(FAKE, 0, 64, 64, FAKE, 0, FAKE, FAKE, FAKE, None, None) == splice.OK              # R = 0


def test_select_argument_errors(L):
    s = L.splice_select_channels
    cnt = ctypes.c_int64(0)
    assert s(FAKE, 16, 64, 64, 65, ctypes.byref(cnt), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) \
        == splice.ERR_INVALID_ARG                                   # k > K
    assert s(FAKE, 16, 64, 64, 4, None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) \
        == splice.ERR_INVALID_ARG                                   # count
    assert s(FAKE, 16, 64, 32, 4, ctypes.byref(cnt), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) \
        == splice.ERR_INVALID_ARG                                   # ldx < K
    assert s(FAKE, 16, 64, 64, 4, ctypes.byref(cnt), FAKE, FAKE, FAKE, None, None, None, 0, None) \
        == splice.ERR_INVALID_ARG                                   # idx
    neg = ctypes.c_int64(-3)
    assert s(FAKE, 16, 64, 64, 4, ctypes.byref(neg), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) \
        == splice.ERR_INVALID_ARG
    assert L.splice_select_workspace_size(4096) == 0


def test_alpha_argument_errors(L):
    a = L.splice_compute_alpha
    need = L.splice_alpha_workspace_size()
    assert need > 0
    assert a(FAKE, 4, 64, 64, FAKE, 0, FAKE, None, 0, None) == splice.ERR_WORKSPACE
    assert a(FAKE, 4, 64, 64, FAKE, 0, FAKE, FAKE, need - 4, None) == splice.ERR_WORKSPACE
    assert a(FAKE, 4, 64, 64, FAKE, 0, None, FAKE, need, None) == splice.ERR_INVALID_ARG
    assert a(FAKE, 4, 60, 64, FAKE, 0, FAKE, FAKE, need, None) == splice.ERR_INVALID_ARG


def test_grouped_argument_errors(L):
    G = splice._Group
    arr = (G * 2)()
    arr[0] = G(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE)
    arr[1] = G(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None)     # no Y
    assert L.splice_gemm_grouped(arr, 2, 64, 256, 8, None, 0, None) == splice.ERR_INVALID_ARG
    assert L.splice_gemm_grouped(arr, 0, 64, 256, 8, None, 0, None) == splice.OK
    assert L.splice_gemm_grouped(None, 2, 64, 256, 8, None, 0, None) == splice.ERR_INVALID_ARG
    empty = (G * 1)()
    empty[0] = G(None, None, None, None, None, None, None, None, 0, None)    # M = 0 group
    assert L.splice_gemm_grouped(empty, 1, 64, 256, 8, None, 0, None) == splice.OK


def test_multi_argument_errors(L):
    S = splice._Seg
    good = S(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 64)

    def call(segs, n, M=4, K=256, k=8, path=0, XS=FAKE):
        return L.splice_gemm_multi(FAKE, FAKE, FAKE, XS, M, K, k, segs, n, None, 0, path, None)
    one = (S * 1)(good)
    assert call(one, 0) == splice.ERR_INVALID_ARG                       # no segment
    assert call(one, splice.SEG_MAX + 1) == splice.ERR_INVALID_ARG      # too many
    assert call(None, 1) == splice.ERR_INVALID_ARG
    two = (S * 2)(good, S(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 32))        # ldy < N
    assert call(two, 2) == splice.ERR_INVALID_ARG
    two = (S * 2)(good, S(FAKE, FAKE, None, FAKE, 64, FAKE, 64))        # no alpha_w
    assert call(two, 2) == splice.ERR_INVALID_ARG
    two = (S * 2)(good, S(FAKE + 4, FAKE, FAKE, FAKE, 64, FAKE, 64))    # misaligned codes
    assert call(two, 2) == splice.ERR_INVALID_ARG
    two = (S * 2)(good, S(FAKE, FAKE + 8, FAKE, FAKE, 64, FAKE, 64))    # scales 8-byte aligned
    assert call(two, 2) == splice.ERR_INVALID_ARG
    assert call(one, 1, XS=None) == splice.ERR_INVALID_ARG               # k > 0 without X_S
    assert call(one, 1, K=144) == splice.ERR_UNSUPPORTED
    assert call(one, 1, M=65, path=splice.PATH_DECODE) == splice.ERR_INVALID_ARG
    assert call(one, 1, M=0) == splice.OK                                # nothing to do
    empty = (S * 2)(S(None, None, None, None, 0, None, 0), S(None, None, None, None, 0, None, 0))
    assert call(empty, 2) == splice.OK                                   # zero widths


def test_fused_multi_argument_errors(L):
    S = splice._Seg
    good = S(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 64)

    def call(segs, n, M=1, K=1024, k=8, X=FAKE, ldx=1024):
        return L.splice_gemm_decode_fused_multi(X, ldx, FAKE, FAKE, M, K, k, segs, n, None)
    one = (S * 1)(good)
    assert call(one, 0) == splice.ERR_INVALID_ARG
    assert call(one, splice.SEG_MAX + 1) == splice.ERR_INVALID_ARG
    assert call(None, 1) == splice.ERR_INVALID_ARG
    assert call(one, 1, M=splice.FUSED_MAX_M + 1) == splice.ERR_UNSUPPORTED
    assert call(one, 1, X=None) == splice.ERR_INVALID_ARG
    assert call(one, 1, ldx=1000) == splice.ERR_INVALID_ARG
    assert call(one, 1, K=1040, ldx=1040) == splice.ERR_UNSUPPORTED     # K % 128
    two = (S * 2)(good, S(FAKE, FAKE, FAKE, None, 64, FAKE, 64))        # k > 0 without W_S
    assert call(two, 2) == splice.ERR_INVALID_ARG
    two = (S * 2)(good, S(FAKE, FAKE + 8, FAKE, FAKE, 64, FAKE, 64))    # scales 8-byte aligned
    assert call(two, 2) == splice.ERR_INVALID_ARG
    assert call(one, 1, M=0) == splice.OK


def fused(L, M=1, N=64, K=1024, k=8, **over):
    args = dict(X=FAKE, ldx=K, idx=FAKE, ax=FAKE, Wq=FAKE, Ws=FAKE, aw=FAKE, WS=FAKE, Y=FAKE,
                ldy=N)
    args.update(over)
    return L.splice_gemm_decode_fused(args["X"], args["ldx"], args["idx"], args["ax"], args["Wq"],
                                      args["Ws"], args["aw"], args["WS"], M, N, K, k, args["Y"],
                                      args["ldy"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), splice.ERR_INVALID_ARG),
    (dict(K=100), splice.ERR_INVALID_ARG),                 # K % 16
    (dict(k=2000), splice.ERR_INVALID_ARG),                # k > K
    (dict(M=splice.FUSED_MAX_M + 1), splice.ERR_UNSUPPORTED),
    (dict(K=400), splice.ERR_UNSUPPORTED),                 # not whole 128-channel chunks
    (dict(K=32768, k=8), splice.ERR_UNSUPPORTED),          # beyond 16 waves x 8 chunks
    (dict(ldx=1028, K=1024), splice.ERR_UNSUPPORTED),      # ldx % 8
    (dict(X=FAKE + 2), splice.ERR_UNSUPPORTED),            # X rows not 16-byte aligned
    (dict(ldx=512), splice.ERR_INVALID_ARG),               # ldx < K
    (dict(X=None), splice.ERR_INVALID_ARG),
    (dict(idx=None), splice.ERR_INVALID_ARG),
    (dict(WS=None), splice.ERR_INVALID_ARG),
    (dict(ax=None), splice.ERR_INVALID_ARG),
    (dict(Y=None), splice.ERR_INVALID_ARG),
    (dict(ldy=10), splice.ERR_INVALID_ARG),
    (dict(Wq=FAKE + 4), splice.ERR_INVALID_ARG),           # misaligned codes
    (dict(Ws=FAKE + 8), splice.ERR_INVALID_ARG),           # scales are loaded as 16-byte vectors
    (dict(idx=FAKE + 2), splice.ERR_INVALID_ARG),
])
def test_fused_decode_argument_errors(L, kw, code):
    assert fused(L, **kw) == code


def test_fused_decode_empty_is_ok(L):
    assert fused(L, M=0) == splice.OK
    assert fused(L, N=0) == splice.OK
    assert fused(L, M=0, K=400) == splice.OK               # nothing to compute: no shape rule applies


def test_channel_stats_argument_errors(L):
    f = L.splice_channel_stats
    cnt = ctypes.c_int64(0)
    assert f(FAKE, -1, 64, 64, ctypes.byref(cnt), FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 64, None, FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG      # count
    assert f(FAKE, 4, 60, 64, ctypes.byref(cnt), FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 32, ctypes.byref(cnt), FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 64, ctypes.byref(cnt), None, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 64, ctypes.byref(cnt), FAKE + 4, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(FAKE, 4, 131072, 131072, ctypes.byref(cnt), FAKE, FAKE, FAKE, None) == splice.ERR_UNSUPPORTED
    bad = ctypes.c_int64(-1)
    assert f(FAKE, 4, 64, 64, ctypes.byref(bad), FAKE, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert cnt.value == 0                                   # nothing folded on an error
    assert f(None, 5, 0, 0, ctypes.byref(cnt), None, None, None, None) == splice.OK
    assert cnt.value == 5                                   # K = 0: rows counted, nothing else


def test_select_topk_argument_errors(L):
    f = L.splice_select_topk
    V, SM = splice.SELECT_VARIANCE, splice.SELECT_SECOND_MOMENT
    assert f(FAKE, FAKE, FAKE, -1, 64, 8, V, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # count
    assert f(FAKE, FAKE, FAKE, 10, 64, 65, V, FAKE, FAKE, None) == splice.ERR_INVALID_ARG  # k > K
    assert f(FAKE, FAKE, FAKE, 10, 60, 8, V, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # K % 16
    assert f(FAKE, FAKE, FAKE, 10, 64, 8, 2, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # criterion
    assert f(None, FAKE, FAKE, 10, 64, 8, SM, FAKE, FAKE, None) == splice.ERR_INVALID_ARG  # mean
    assert f(FAKE, None, FAKE, 10, 64, 8, V, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # m2
    assert f(FAKE, FAKE, None, 10, 64, 8, V, FAKE, FAKE, None) == splice.ERR_INVALID_ARG   # absmax
    assert f(FAKE, FAKE, FAKE, 10, 64, 8, V, None, FAKE, None) == splice.ERR_INVALID_ARG   # idx
    assert f(FAKE, FAKE + 4, FAKE, 10, 64, 8, V, FAKE, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(None, None, None, 10, 0, 0, SM, None, None, None) == splice.OK                # K = 0


def test_tim_filter_argument_errors(L):
    f = L.splice_tim_filter
    ok = (FAKE, 4, 64, FAKE, -9.0, 1, 100, 5, FAKE, FAKE, FAKE, FAKE, 1, 1, None)

    def call(**over):
        a = list(ok)
        names = ["logp", "B", "ldl", "len", "tau", "k1n", "k1d", "k2", "keep", "g1", "g2", "adv",
                 "cols", "lda", "s"]
        for k, v in over.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(B=-1) == splice.ERR_INVALID_ARG
    assert call(k1d=0) == splice.ERR_INVALID_ARG
    assert call(k1n=-1) == splice.ERR_INVALID_ARG
    assert call(k2=-1) == splice.ERR_INVALID_ARG
    assert call(len=None) == splice.ERR_INVALID_ARG
    assert call(logp=None) == splice.ERR_INVALID_ARG
    assert call(adv=None) == splice.ERR_INVALID_ARG          # cols > 0 without adv
    assert call(cols=8, lda=4) == splice.ERR_INVALID_ARG     # lda < cols
    assert call(g1=FAKE + 2) == splice.ERR_INVALID_ARG
    assert call(B=1 << 31) == splice.ERR_UNSUPPORTED
    assert call(B=0) == splice.OK                            # nothing to do


def test_probe_argument_errors(L):
    f = L.splice_probe_mfma_f16
    assert f(-1, 8, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(16, 0, FAKE, None) == splice.ERR_INVALID_ARG
    assert f(16, 8, None, None) == splice.ERR_INVALID_ARG
    assert f(16, 8, FAKE + 2, None) == splice.ERR_INVALID_ARG
    r = L.splice_probe_stream_read
    assert r(FAKE, 100, 8, FAKE, None) == splice.ERR_INVALID_ARG       # not a multiple of 16
    assert r(FAKE, -16, 8, FAKE, None) == splice.ERR_INVALID_ARG
    assert r(FAKE, 1 << 20, 0, FAKE, None) == splice.ERR_INVALID_ARG
    assert r(FAKE + 8, 1 << 20, 8, FAKE, None) == splice.ERR_INVALID_ARG  # misaligned source
    assert r(None, 1 << 20, 8, FAKE, None) == splice.ERR_INVALID_ARG
    assert r(FAKE, 1 << 20, 8, None, None) == splice.ERR_INVALID_ARG


LOG_PROBE = """
import ctypes
from fp4_gemm_sparse_amd import splice
L = splice.lib()
F = 0x100000
def gemm(M, N, K, k, path):
    return L.splice_gemm(F, F, F, F, F, F, F, F, M, N, K, k, F, N, None, 0, path, None)
print(gemm(128, 1024, 4096, 64, splice.PATH_AUTO), gemm(64, 1024, 4096, 64, splice.PATH_DECODE),
      gemm(8, 64, 100, 8, splice.PATH_AUTO))
"""


@pytest.mark.parametrize("flag", ["1", "0", None])
def test_splice_log_lines(flag):
    """SPLICE_LOG: one stderr line per GEMM call that passes its argument
    checks, with the plan it chose and its status; nothing when unset or 0."""
    import os
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("SPLICE_LOG", None)
    if flag is not None:
        env["SPLICE_LOG"] = flag
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", LOG_PROBE], capture_output=True, text=True, env=env, cwd=root,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == [str(splice.ERR_WORKSPACE), str(splice.ERR_WORKSPACE), str(splice.ERR_INVALID_ARG)]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[splice]")]
    if flag != "1":
        assert lines == []
        return
    assert len(lines) == 2, r.stderr
    assert "splice_gemm M=128 N=1024 K=4096 k=64 segments=0 path=prefill" in lines[0]
    assert "tile=128x128 splits=8 status=-3" in lines[0]
    assert "M=64 N=1024 K=4096 k=64 segments=0 path=decode" in lines[1]
    assert "tile=64x32 splits=4 status=-3" in lines[1]


ROCTX_PROBE = LOG_PROBE + """
with open("/proc/self/maps") as f:
    print(int(any("rocprofiler-sdk-roctx" in line for line in f)))
"""


@pytest.mark.parametrize("flag", ["1", "0", None])
def test_splice_roctx_ranges(flag):
    """SPLICE_ROCTX: the library opens ROCm's roctx library at its first
    call only when the flag is set (torch maps a roctx library of its own, so
    the check names ROCm's), and the ranges leave every status as it was."""
    import os
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("SPLICE_ROCTX", None)
    env.pop("SPLICE_LOG", None)
    if flag is not None:
        env["SPLICE_ROCTX"] = flag
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", ROCTX_PROBE], capture_output=True, text=True, env=env, cwd=root,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    out = r.stdout.split()
    assert out[:3] == [str(splice.ERR_WORKSPACE), str(splice.ERR_WORKSPACE), str(splice.ERR_INVALID_ARG)]
    assert out[3] == ("1" if flag == "1" else "0"), r.stdout
