"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/ttq.h declares, and rejects malformed arguments on the host
before any HIP call (fake, never-dereferenced device addresses are used)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ttq.h")
LIBPATH = os.path.join(ROOT, "online_activation_aware_amd", "libttq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIBPATH), reason="libttq.so not built")

FAKE = 0x100000  # 1 MiB: 256-byte aligned, never dereferenced by the failing calls


@pytest.fixture(scope="module")
def L():
    from online_activation_aware_amd import ttq
    return ttq.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_all_exported(L):
    from online_activation_aware_amd import ttq
    names = header_functions()
    assert set(names) == set(ttq.EXPORTS)
    raw = ctypes.CDLL(LIBPATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(L):
    assert L.ttq_status_str(0) == b"TTQ_OK"
    assert L.ttq_status_str(1) == b"TTQ_ERR_INVALID"
    assert L.ttq_status_str(2) == b"TTQ_ERR_UNSUPPORTED"
    assert L.ttq_status_str(3) == b"TTQ_ERR_DEVICE"
    assert L.ttq_status_str(99) == b"TTQ_ERR_UNKNOWN"


def test_workspace_bytes(L):
    from online_activation_aware_amd import ttq
    n = ttq.ttq_workspace_bytes(2048, 4096, 4096, 4, 32, 0)
    # at least the quantization state: ssq + s + codes + steps + zeros
    state = 4096 * 8 + 4096 * 4 + 4096 * 4096 * 4 // 8 + 2 * 4096 * 128 * 2
    assert n >= state and n % 256 == 0
    # prompt-sized projections stage the dequantized weight (M x K bf16)
    assert n >= state + 4096 * 4096 * 2
    assert ttq.ttq_workspace_bytes(16, 4096, 4096, 4, 32, 0) < state + 4096 * 4096 * 2
    assert ttq.ttq_workspace_bytes(2048, 4096, 4096, 2, 32, 16) >= ttq.ttq_workspace_bytes(2048, 4096, 4096, 2, 32, 0)
    # 14336 -> 4096 at T = 1024 has 128 output tiles of 128 x 256: the GEMM
    # runs as two K slices, whose fp32 partials follow the dequantized weight
    T, K, M = 1024, 14336, 4096
    st4 = K * 8 + K * 4 + M * K * 4 // 8 + 2 * M * (K // 32) * 2
    n4 = ttq.ttq_workspace_bytes(T, K, M, 4, 32, 0)
    assert n4 >= st4 + M * K * 2 + 2 * T * M * 4
    # with 256 or more tiles (T = 2048 here) no partials are needed
    assert ttq.ttq_workspace_bytes(2048, K, M, 4, 32, 0) < st4 + M * K * 2 + 2 * 2048 * M * 4
    # ragged M: the partial rows are padded to a multiple of 4 floats
    assert ttq.ttq_workspace_bytes(300, 8192, 130, 4, 32, 0) >= 8192 * 130 * 2 + 2 * 300 * 132 * 4
    for bad in [(10, 100, 10, 4, 32, 0),     # K not a multiple of 32
                (10, 128, 10, 6, 32, 0),     # bits
                (10, 128, 10, 4, 48, 0),     # group
                (10, 96, 10, 4, 64, 0),      # group does not divide K
                (10, 128, 10, 4, 32, 65),    # rank
                (-1, 128, 10, 4, 32, 0)]:
        assert ttq.ttq_workspace_bytes(*bad) == 0


def _err(L):
    return L.ttq_last_error().decode()


def test_stats_rejects(L):
    st = L.ttq_stats
    assert st(FAKE, 1, 16, 100, 100, FAKE, 0, FAKE, 1 << 30, None) == 1   # K % 8
    assert "K" in _err(L)
    assert st(FAKE, 5, 16, 128, 128, FAKE, 0, FAKE, 1 << 30, None) == 1   # dtype
    assert st(FAKE, 1, 16, 128, 64, FAKE, 0, FAKE, 1 << 30, None) == 1    # ldx < K
    assert st(FAKE + 2, 1, 16, 128, 128, FAKE, 0, FAKE, 1 << 30, None) == 1  # X alignment
    assert st(FAKE, 1, 16, 128, 132, FAKE, 0, FAKE, 1 << 30, None) == 1   # stride bytes
    assert st(None, 1, 16, 128, 128, FAKE, 0, FAKE, 1 << 30, None) == 1   # null X
    assert st(FAKE, 1, 16, 128, 128, None, 0, FAKE, 1 << 30, None) == 1   # null ssq
    sp = L.ttq_stats_p
    assert sp(FAKE, 1, 16, 128, 128, 0.0, FAKE, 0, FAKE, 1 << 30, None) == 1   # p <= 0
    assert "p must be finite" in _err(L)
    assert sp(FAKE, 1, 16, 128, 128, float("nan"), FAKE, 0, FAKE, 1 << 30, None) == 1
    assert sp(FAKE, 1, 16, 100, 100, 1.0, FAKE, 0, FAKE, 1 << 30, None) == 1   # K % 8


def test_scales_rejects(L):
    sc = L.ttq_awq_scales
    assert sc(FAKE, 0, 128, 0.5, 0.01, 2.0, FAKE, None) == 1               # n_tokens
    assert sc(FAKE, 4, 128, -0.5, 0.01, 2.0, FAKE, None) == 1              # alpha < 0
    assert sc(FAKE, 4, 128, float("nan"), 0.01, 2.0, FAKE, None) == 1      # alpha NaN
    assert sc(FAKE, 4, 128, 0.5, float("inf"), 2.0, FAKE, None) == 1       # lambda
    assert sc(FAKE, 4, 128, 0.5, 0.01, 0.0, FAKE, None) == 1               # p <= 0
    assert "p must be finite" in _err(L)
    assert sc(FAKE, 4, 128, 0.5, 0.01, float("nan"), FAKE, None) == 1      # p NaN
    assert sc(FAKE, 4, 128, 0.5, 0.01, 2.0, FAKE + 4, None) == 1           # s alignment


def test_quantize_rejects(L):
    q = L.ttq_quantize_groups
    ok = dict(W=FAKE, wt=1, M=64, K=256, ldw=256, s=FAKE, bits=4, group=32, B=None, A=None, rank=0,
              codes=FAKE, scale=FAKE, zero=FAKE, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return q(*a.values())
    assert call(bits=1) == 1 and call(bits=6) == 1
    assert call(group=8) == 1 and call(group=256) == 1
    assert call(K=96, ldw=96, group=64) == 1           # group does not divide K
    assert call(K=48, ldw=48, group=16) == 1           # K not a multiple of 32
    assert call(rank=4) == 1                           # rank without factors
    assert call(rank=0, B=FAKE, A=FAKE) == 1           # factors without rank
    assert call(rank=65, B=FAKE, A=FAKE) == 1          # rank above the limit
    assert call(codes=None) == 1
    assert call(s=FAKE + 4) == 1
    assert call(M=-1) == 1
    assert call(M=0) == 0                               # empty: nothing to do


def test_qgemm_rejects(L):
    g = L.ttq_qgemm
    ok = dict(X=FAKE, xt=1, T=8, K=256, ldx=256, s=FAKE, codes=FAKE, scale=FAKE, zero=FAKE, M=64,
              bits=4, group=32, Y=FAKE, yt=0, ldy=64, ws=FAKE, wsb=1 << 20, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(*a.values())
    assert call(ldy=32) == 1                            # ldy < M
    assert call(Y=FAKE + 2) == 1                        # fp32 Y not 4-byte aligned
    assert call(ldx=260) == 1                           # X rows (520 B) not a multiple of 16 bytes
    assert call(s=None) == 1
    assert call(codes=FAKE + 4) == 1                    # codes not 16-byte aligned
    assert call(bits=1) == 1
    assert call(yt=7) == 1
    assert call(T=0) == 0 and call(M=0) == 0            # empty calls


def test_lowrank_and_linear_reject(L):
    from online_activation_aware_amd import ttq
    assert L.ttq_lowrank_add(FAKE, 1, 8, 256, 256, FAKE, FAKE, 64, 0, FAKE, 0, 64, FAKE, 1 << 20, None) == 1
    assert L.ttq_lowrank_add(FAKE, 1, 8, 256, 256, None, FAKE, 64, 4, FAKE, 0, 64, FAKE, 1 << 20, None) == 1
    assert L.ttq_linear(None, FAKE, 1 << 20, None) == 1
    a = ttq.LinearArgs(X=FAKE, xt=1, T=8, K=256, ldx=256, W=FAKE, wt=1, M=64, ldw=256, alpha=0.5,
                       lambda_rel=0.01, p=0.0, bits=4, group=32, B=None, A=None, rank=0, Y=FAKE, yt=0,
                       ldy=64)
    assert L.ttq_linear(ctypes.byref(a), FAKE, 1 << 30, None) == 1   # p <= 0
    a.p = float("inf")
    assert L.ttq_linear(ctypes.byref(a), FAKE, 1 << 30, None) == 1   # p not finite
    a.p = 2.0
    a.bits = 9
    assert L.ttq_linear(ctypes.byref(a), FAKE, 1 << 30, None) == 1
    a.bits = 4
    assert L.ttq_linear(ctypes.byref(a), FAKE, 16, None) == 1         # workspace too small
    handles = (ctypes.c_void_p * ttq.TTQ_LINEAR_STAGE_EVENTS)(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE)
    a.stage_events = ctypes.cast(handles, ctypes.c_void_p)
    assert L.ttq_linear(ctypes.byref(a), FAKE, 1 << 30, None) == 1    # a null event handle
    assert "stage_events" in _err(L)
    a.stage_events = None
    a.T = 0
    assert L.ttq_linear(ctypes.byref(a), None, 0, None) == 0          # empty prompt


def test_lowrank_factors_rejects(L):
    f = L.ttq_lowrank_factors
    ok = dict(W=FAKE, wt=1, M=256, K=512, ldw=512, s=FAKE, om=FAKE, l=24, q=2, rank=16, B=FAKE, A=FAKE,
              ws=FAKE, wn=1 << 30, st=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["W"], a["wt"], a["M"], a["K"], a["ldw"], a["s"], a["om"], a["l"], a["q"], a["rank"],
                 a["B"], a["A"], a["ws"], a["wn"], a["st"])
    assert call(K=500, ldw=500) == 1                    # K % 32
    assert call(l=33) == 1 and call(l=0) == 1
    assert call(rank=25) == 1 and call(rank=0) == 1     # rank <= l
    assert call(M=16) == 1                              # l <= M
    assert call(q=-1) == 1
    assert call(s=None) == 1 and call(om=None) == 1 and call(B=None) == 1
    assert call(wt=0) == 2                              # fp32 weight: not implemented
    assert call(wn=64) == 1                             # workspace too small
    assert "workspace" in _err(L)
    assert L.ttq_lowrank_factors_workspace_bytes(256, 512, 24) > 256 * 512 * 2
    assert L.ttq_lowrank_factors_workspace_bytes(256, 512, 40) == 0


def test_qgemm_batched_rejects(L):
    f = L.ttq_qgemm_batched
    ok = dict(X=FAKE, xt=1, P=3, T=1, K=1024, ldx=1024, xs=1024, s=FAKE, ss=1024, c=FAKE, cst=512, sc=FAKE,
              z=FAKE, szs=32, M=64, bits=4, group=32, Y=FAKE, yt=0, ldy=64, ys=64)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["X"], a["xt"], a["P"], a["T"], a["K"], a["ldx"], a["xs"], a["s"], a["ss"], a["c"], a["cst"],
                 a["sc"], a["z"], a["szs"], a["M"], a["bits"], a["group"], a["Y"], a["yt"], a["ldy"], a["ys"], None)
    assert call(T=5) == 1 and call(T=0) == 1             # batched steps: 1 <= T <= 4
    assert call(P=0) == 1
    assert call(K=1056, ldx=1056, xs=1056) == 1          # K % 128
    assert call(xs=1000) == 1                            # prompts' X overlap
    assert call(xs=1028) == 1                            # X stride not 16-byte aligned for bf16
    assert call(ss=2) == 1 and call(cst=6) == 1          # s / codes strides break 16-byte alignment
    assert call(ys=10) == 1                              # prompts' Y overlap
    assert call(s=None) == 1


def test_linear_shared_rejects(L):
    from online_activation_aware_amd import ttq
    arr = (ttq.LinearArgs * 2)()
    for i in range(2):
        arr[i] = ttq.LinearArgs(X=FAKE, xt=1, T=8, K=256, ldx=256, W=FAKE, wt=1, M=64, ldw=256, alpha=0.5,
                                lambda_rel=0.01, p=2.0, bits=4, group=32, B=None, A=None, rank=0, Y=FAKE, yt=0,
                                ldy=64)
    assert L.ttq_linear_shared(arr, 0, FAKE, 1 << 30, None) == 1          # n
    assert L.ttq_linear_shared_workspace_bytes(arr, 2) > 0
    arr[1].ldx = 512
    assert L.ttq_linear_shared(arr, 2, FAKE, 1 << 30, None) == 1          # different input
    assert "layer 1" in _err(L)
    arr[1].ldx = 256
    arr[1].alpha = 0.25
    assert L.ttq_linear_shared(arr, 2, FAKE, 1 << 30, None) == 1          # different alpha
    arr[1].alpha = 0.5
    arr[1].ssq = FAKE
    assert L.ttq_linear_shared(arr, 2, FAKE, 1 << 30, None) == 1          # ssq only on layer 0
    arr[1].ssq = None
    assert L.ttq_linear_shared(arr, 2, FAKE, 64, None) == 1               # workspace too small
