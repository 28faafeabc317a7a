"""Thin ctypes binding of libttq (include/ttq.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libttq.so.  Tensors must be device (HIP) tensors; PyTorch supplies memory and
the current stream.  There is no CPU fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttq.so")

TTQ_OK, TTQ_ERR_INVALID, TTQ_ERR_UNSUPPORTED, TTQ_ERR_DEVICE = 0, 1, 2, 3
TTQ_F32, TTQ_BF16 = 0, 1

EXPORTS = ("ttq_stats", "ttq_stats_p", "ttq_awq_scales", "ttq_quantize_groups", "ttq_qgemm", "ttq_qgemm_batched",
           "ttq_lowrank_add", "ttq_lowrank_factors", "ttq_lowrank_factors_workspace_bytes",
           "ttq_workspace_bytes", "ttq_linear", "ttq_linear_shared", "ttq_linear_shared_workspace_bytes",
           "ttq_linear_noalloc", "ttq_status_str", "ttq_last_error")


class TTQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class LinearArgs(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p), ("xt", ctypes.c_int), ("T", ctypes.c_int64),
        ("K", ctypes.c_int64), ("ldx", ctypes.c_int64),
        ("W", ctypes.c_void_p), ("wt", ctypes.c_int), ("M", ctypes.c_int64),
        ("ldw", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("lambda_rel", ctypes.c_float), ("p", ctypes.c_float),
        ("bits", ctypes.c_int), ("group", ctypes.c_int),
        ("B", ctypes.c_void_p), ("A", ctypes.c_void_p), ("rank", ctypes.c_int),
        ("Y", ctypes.c_void_p), ("yt", ctypes.c_int), ("ldy", ctypes.c_int64),
        ("ssq", ctypes.c_void_p), ("s", ctypes.c_void_p), ("codes", ctypes.c_void_p),
        ("scale_f16", ctypes.c_void_p), ("zero_f16", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
    ]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libttq.so (once) and declare the C signatures."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m online_activation_aware_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "ttq_stats": [vp, i32, i64, i64, i64, vp, i32, vp, sz, vp],
        "ttq_stats_p": [vp, i32, i64, i64, i64, f32, vp, i32, vp, sz, vp],
        "ttq_awq_scales": [vp, i64, i64, f32, f32, f32, vp, vp],
        "ttq_quantize_groups": [vp, i32, i64, i64, i64, vp, i32, i32, vp, vp, i32, vp, vp, vp, vp],
        "ttq_qgemm": [vp, i32, i64, i64, i64, vp, vp, vp, vp, i64, i32, i32, vp, i32, i64, vp, sz, vp],
        "ttq_lowrank_add": [vp, i32, i64, i64, i64, vp, vp, i64, i32, vp, i32, i64, vp, sz, vp],
        "ttq_qgemm_batched": [vp, i32, i64, i64, i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i64, i32, i32, vp,
                              i32, i64, i64, vp],
        "ttq_workspace_bytes": [i64, i64, i64, i32, i32, i32],
        "ttq_lowrank_factors": [vp, i32, i64, i64, i64, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp],
        "ttq_lowrank_factors_workspace_bytes": [i64, i64, i32],
        "ttq_linear": [ctypes.POINTER(LinearArgs), vp, sz, vp],
        "ttq_linear_noalloc": [ctypes.POINTER(LinearArgs), vp],
        "ttq_linear_shared": [ctypes.POINTER(LinearArgs), i32, vp, sz, vp],
        "ttq_linear_shared_workspace_bytes": [ctypes.POINTER(LinearArgs), i32],
        "ttq_status_str": [i32],
        "ttq_last_error": [],
    }
    for name, argtypes in sig.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    L.ttq_workspace_bytes.restype = ctypes.c_size_t
    L.ttq_lowrank_factors_workspace_bytes.restype = ctypes.c_size_t
    L.ttq_linear_shared_workspace_bytes.restype = ctypes.c_size_t
    L.ttq_status_str.restype = ctypes.c_char_p
    L.ttq_last_error.restype = ctypes.c_char_p
    _lib_handle = L
    return L


# ------------------------------------------------------------------ helpers

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TTQ_F32
    if t.dtype == torch.bfloat16:
        return TTQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    return t.data_ptr()


def _ld(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride in its last dimension")
    return t.stride(0)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _torch_stream(stream) -> torch.cuda.Stream:
    """The launch stream as a torch stream (a raw hipStream_t handle is
    wrapped as an external stream)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _on_launch_stream(fn):
    """Run a call with its launch stream as torch's current stream, so that
    every tensor the binding allocates for it (outputs, default workspaces)
    belongs to the stream the kernels run on: the caching allocator then
    cannot hand such memory to other work before those kernels are done."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def call(*args, **kwargs):
        bound = sig.bind(*args, **kwargs)
        ts = _torch_stream(bound.arguments.get("stream"))
        bound.arguments["stream"] = ts
        with torch.cuda.stream(ts):
            return fn(*bound.args, **bound.kwargs)
    return call


def _check(status: int) -> None:
    if status != TTQ_OK:
        L = lib()
        raise TTQError(status, f"{L.ttq_status_str(status).decode()}: {L.ttq_last_error().decode()}")


def _ws(ws: Optional[torch.Tensor], device) -> tuple:
    if ws is None:
        return None, 0
    if ws.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    return _dev(ws, "ws"), ws.numel()


# ------------------------------------------------------------------ calls

def ttq_workspace_bytes(T: int, K: int, M: int, bits: int, group: int, rank: int = 0) -> int:
    return int(lib().ttq_workspace_bytes(T, K, M, bits, group, rank))


def workspace(T: int, K: int, M: int, bits: int, group: int, rank: int = 0, device="cuda") -> torch.Tensor:
    """Allocate a workspace tensor of ttq_workspace_bytes() bytes."""
    n = ttq_workspace_bytes(T, K, M, bits, group, rank)
    if n == 0:
        raise ValueError("no call accepts these sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


@_on_launch_stream
def ttq_stats(X: torch.Tensor, ssq: torch.Tensor, accumulate: bool = False,
              ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if ssq.dtype != torch.float64:
        raise TypeError("ssq must be float64")
    T, K = X.shape
    wp, wn = _ws(ws, X.device)
    _check(lib().ttq_stats(_dev(X, "X"), _dtype_code(X), T, K, _ld(X, "X"), _dev(ssq, "ssq"),
                           int(bool(accumulate)), wp, wn, _stream(stream)))
    return ssq


@_on_launch_stream
def ttq_stats_p(X: torch.Tensor, p: float, msum: torch.Tensor, accumulate: bool = False,
                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if msum.dtype != torch.float64:
        raise TypeError("msum must be float64")
    T, K = X.shape
    wp, wn = _ws(ws, X.device)
    _check(lib().ttq_stats_p(_dev(X, "X"), _dtype_code(X), T, K, _ld(X, "X"), p, _dev(msum, "msum"),
                             int(bool(accumulate)), wp, wn, _stream(stream)))
    return msum


@_on_launch_stream
def ttq_awq_scales(ssq: torch.Tensor, n_tokens: int, alpha: float, lambda_rel: float,
                   p: float = 2.0, s: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    K = ssq.numel()
    if s is None:
        s = torch.empty(K, dtype=torch.float32, device=ssq.device)
    _check(lib().ttq_awq_scales(_dev(ssq, "ssq"), n_tokens, K, alpha, lambda_rel, p, _dev(s, "s"),
                                _stream(stream)))
    return s


@_on_launch_stream
def ttq_quantize_groups(W: torch.Tensor, s: Optional[torch.Tensor], bits: int, group: int,
                        B: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                        codes: Optional[torch.Tensor] = None, scale_f16: Optional[torch.Tensor] = None,
                        zero_f16: Optional[torch.Tensor] = None, stream=None):
    M, K = W.shape
    rank = 0 if B is None else B.shape[1]
    dev = W.device
    if codes is None:
        codes = torch.empty((M, K * bits // 32), dtype=torch.int32, device=dev)
    if scale_f16 is None:
        scale_f16 = torch.empty((M, K // group), dtype=torch.float16, device=dev)
    if zero_f16 is None:
        zero_f16 = torch.empty((M, K // group), dtype=torch.float16, device=dev)
    _check(lib().ttq_quantize_groups(_dev(W, "W"), _dtype_code(W), M, K, _ld(W, "W"), _dev(s, "s"),
                                     bits, group, _dev(B, "B"), _dev(A, "A"), rank, _dev(codes, "codes"),
                                     _dev(scale_f16, "scale_f16"), _dev(zero_f16, "zero_f16"),
                                     _stream(stream)))
    return codes, scale_f16, zero_f16


@_on_launch_stream
def ttq_qgemm(X: torch.Tensor, s: torch.Tensor, codes: torch.Tensor, scale_f16: torch.Tensor,
              zero_f16: torch.Tensor, M: int, bits: int, group: int, Y: Optional[torch.Tensor] = None,
              y_dtype=torch.float32, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, K = X.shape
    if Y is None:
        Y = torch.empty((T, M), dtype=y_dtype, device=X.device)
    wp, wn = _ws(ws, X.device)
    _check(lib().ttq_qgemm(_dev(X, "X"), _dtype_code(X), T, K, _ld(X, "X"), _dev(s, "s"),
                           _dev(codes, "codes"), _dev(scale_f16, "scale_f16"), _dev(zero_f16, "zero_f16"),
                           M, bits, group, _dev(Y, "Y"), _dtype_code(Y), _ld(Y, "Y"), wp, wn,
                           _stream(stream)))
    return Y


@_on_launch_stream
def ttq_qgemm_batched(X: torch.Tensor, s: torch.Tensor, codes: torch.Tensor, scale_f16: torch.Tensor,
                      zero_f16: torch.Tensor, M: int, bits: int, group: int, Y: Optional[torch.Tensor] = None,
                      y_dtype=torch.float32, stream=None) -> torch.Tensor:
    """One decode step of P prompts: X [P][T][K], s [P][K], codes [P][M][.],
    scale_f16 / zero_f16 [P][M][K/group]; returns Y [P][T][M]."""
    P, T, K = X.shape
    if Y is None:
        Y = torch.empty((P, T, M), dtype=y_dtype, device=X.device)
    for name, t in (("s", s), ("codes", codes), ("scale_f16", scale_f16), ("zero_f16", zero_f16)):
        if t.shape[0] != P or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous [P][...] tensor")
    if X.stride(2) != 1 or Y.stride(2) != 1:
        raise ValueError("X and Y rows must be contiguous")
    if scale_f16.stride(0) != zero_f16.stride(0):
        raise ValueError("scale_f16 and zero_f16 must have the same prompt stride")
    _check(lib().ttq_qgemm_batched(_dev(X, "X"), _dtype_code(X), P, T, K, X.stride(1), X.stride(0),
                                   _dev(s, "s"), s.stride(0), _dev(codes, "codes"), codes.stride(0),
                                   _dev(scale_f16, "scale_f16"), _dev(zero_f16, "zero_f16"), scale_f16.stride(0),
                                   M, bits, group, _dev(Y, "Y"), _dtype_code(Y), Y.stride(1), Y.stride(0),
                                   _stream(stream)))
    return Y


@_on_launch_stream
def ttq_lowrank_add(X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, Y: torch.Tensor,
                    ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, K = X.shape
    M, rank = B.shape
    wp, wn = _ws(ws, X.device)
    _check(lib().ttq_lowrank_add(_dev(X, "X"), _dtype_code(X), T, K, _ld(X, "X"), _dev(A, "A"),
                                 _dev(B, "B"), M, rank, _dev(Y, "Y"), _dtype_code(Y), _ld(Y, "Y"),
                                 wp, wn, _stream(stream)))
    return Y


@_on_launch_stream
def ttq_lowrank_factors(W: torch.Tensor, s: torch.Tensor, omega: torch.Tensor, rank: int, q: int,
                        B: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None):
    """Per-prompt factors of W diag(s): returns (B [M][rank], A [rank][K])."""
    M, K = W.shape
    l = omega.shape[0]
    if omega.shape != (l, K) or omega.dtype != torch.float32:
        raise ValueError("omega must be float32 [l][K]")
    if B is None:
        B = torch.empty((M, rank), dtype=torch.float32, device=W.device)
    if A is None:
        A = torch.empty((rank, K), dtype=torch.float32, device=W.device)
    if ws is None:
        n = lib().ttq_lowrank_factors_workspace_bytes(M, K, l)
        if n == 0:
            raise ValueError("no factorization accepts these sizes")
        ws = torch.empty(n, dtype=torch.uint8, device=W.device)
    _check(lib().ttq_lowrank_factors(_dev(W, "W"), _dtype_code(W), M, K, _ld(W, "W"), _dev(s, "s"),
                                     _dev(omega, "omega"), l, q, rank, _dev(B, "B"), _dev(A, "A"),
                                     ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))
    return B, A


@_on_launch_stream
def ttq_linear(X: torch.Tensor, W: torch.Tensor, bits: int, group: int, alpha: float,
               lambda_rel: float, p: float = 2.0, B: Optional[torch.Tensor] = None,
               A: Optional[torch.Tensor] = None, Y: Optional[torch.Tensor] = None,
               y_dtype=torch.float32, ws: Optional[torch.Tensor] = None, state: Optional[dict] = None,
               stream=None, stage_events=None) -> torch.Tensor:
    """One call for the whole layer.  ``state`` may hold preallocated output
    tensors ``ssq``, ``s``, ``codes``, ``scale_f16``, ``zero_f16`` that receive
    the prompt's quantization state (for later decode-step ttq_qgemm calls).
    ``stage_events``: optional StageEvents, recorded at the stage boundaries."""
    T, K = X.shape
    M = W.shape[0]
    rank = 0 if B is None else B.shape[1]
    if Y is None:
        Y = torch.empty((T, M), dtype=y_dtype, device=X.device)
    if ws is None:
        ws = workspace(T, K, M, bits, group, rank, device=X.device)
    st = state or {}
    a = LinearArgs(
        X=_dev(X, "X"), xt=_dtype_code(X), T=T, K=K, ldx=_ld(X, "X"),
        W=_dev(W, "W"), wt=_dtype_code(W), M=M, ldw=_ld(W, "W"),
        alpha=alpha, lambda_rel=lambda_rel, p=p, bits=bits, group=group,
        B=_dev(B, "B"), A=_dev(A, "A"), rank=rank,
        Y=_dev(Y, "Y"), yt=_dtype_code(Y), ldy=_ld(Y, "Y"),
        ssq=_dev(st.get("ssq"), "ssq"), s=_dev(st.get("s"), "s"), codes=_dev(st.get("codes"), "codes"),
        scale_f16=_dev(st.get("scale_f16"), "scale_f16"), zero_f16=_dev(st.get("zero_f16"), "zero_f16"),
        stage_events=None if stage_events is None else ctypes.cast(stage_events.handles, ctypes.c_void_p),
    )
    wp, wn = _ws(ws, X.device)
    _check(lib().ttq_linear(ctypes.byref(a), wp, wn, _stream(stream)))
    return Y


@_on_launch_stream
def ttq_linear_noalloc(X: torch.Tensor, W: torch.Tensor, bits: int, group: int, alpha: float,
                       lambda_rel: float, Y: torch.Tensor, p: float = 2.0, B: Optional[torch.Tensor] = None,
                       A: Optional[torch.Tensor] = None, state: Optional[dict] = None,
                       stream=None) -> torch.Tensor:
    """ttq_linear with the library's own scratch array as the workspace (the
    call allocates nothing; Y and the optional state tensors come from the
    caller)."""
    T, K = X.shape
    M = W.shape[0]
    st = state or {}
    a = LinearArgs(
        X=_dev(X, "X"), xt=_dtype_code(X), T=T, K=K, ldx=_ld(X, "X"),
        W=_dev(W, "W"), wt=_dtype_code(W), M=M, ldw=_ld(W, "W"),
        alpha=alpha, lambda_rel=lambda_rel, p=p, bits=bits, group=group,
        B=_dev(B, "B"), A=_dev(A, "A"), rank=0 if B is None else B.shape[1],
        Y=_dev(Y, "Y"), yt=_dtype_code(Y), ldy=_ld(Y, "Y"),
        ssq=_dev(st.get("ssq"), "ssq"), s=_dev(st.get("s"), "s"), codes=_dev(st.get("codes"), "codes"),
        scale_f16=_dev(st.get("scale_f16"), "scale_f16"), zero_f16=_dev(st.get("zero_f16"), "zero_f16"),
        stage_events=None)
    _check(lib().ttq_linear_noalloc(ctypes.byref(a), _stream(stream)))
    return Y


@_on_launch_stream
def ttq_linear_shared(X: torch.Tensor, layers: list, alpha: float, lambda_rel: float, p: float = 2.0,
                      ws: Optional[torch.Tensor] = None, stream=None) -> list:
    """Several layers on the same X with one statistics pass.  ``layers``:
    dicts with ``W``, ``bits``, ``group`` and optionally ``B``, ``A``, ``Y``,
    ``y_dtype``, ``state`` (only the first layer's state may hold ``ssq``).
    Returns the layers' outputs Y."""
    T, K = X.shape
    arr = (LinearArgs * len(layers))()
    outs = []
    for i, ly in enumerate(layers):
        W = ly["W"]
        M = W.shape[0]
        B, A = ly.get("B"), ly.get("A")
        Y = ly.get("Y")
        if Y is None:
            Y = torch.empty((T, M), dtype=ly.get("y_dtype", torch.float32), device=X.device)
        outs.append(Y)
        st = ly.get("state") or {}
        arr[i] = LinearArgs(
            X=_dev(X, "X"), xt=_dtype_code(X), T=T, K=K, ldx=_ld(X, "X"),
            W=_dev(W, "W"), wt=_dtype_code(W), M=M, ldw=_ld(W, "W"),
            alpha=alpha, lambda_rel=lambda_rel, p=p, bits=ly["bits"], group=ly["group"],
            B=_dev(B, "B"), A=_dev(A, "A"), rank=0 if B is None else B.shape[1],
            Y=_dev(Y, "Y"), yt=_dtype_code(Y), ldy=_ld(Y, "Y"),
            ssq=_dev(st.get("ssq"), "ssq"), s=_dev(st.get("s"), "s"), codes=_dev(st.get("codes"), "codes"),
            scale_f16=_dev(st.get("scale_f16"), "scale_f16"), zero_f16=_dev(st.get("zero_f16"), "zero_f16"),
            stage_events=None)
    if ws is None:
        n = lib().ttq_linear_shared_workspace_bytes(arr, len(layers))
        if n == 0:
            raise ValueError("no call accepts these sizes")
        ws = torch.empty(n, dtype=torch.uint8, device=X.device)
    wp, wn = _ws(ws, X.device)
    _check(lib().ttq_linear_shared(arr, len(layers), wp, wn, _stream(stream)))
    return outs


TTQ_LINEAR_STAGE_EVENTS = 8
LINEAR_STAGES = ("stats", "quantize", "projection", "lowrank")

_hip_handle = None


def _hip() -> ctypes.CDLL:
    """The HIP runtime already loaded by torch (same soname, one runtime)."""
    global _hip_handle
    if _hip_handle is None:
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreate.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip_handle = h
    return _hip_handle


class StageEvents:
    """TTQ_LINEAR_STAGE_EVENTS timing events for ttq_linear(stage_events=...):
    a (start, stop) pair per stage, stamped by the stage's own kernels."""

    def __init__(self):
        h = _hip()
        self.handles = (ctypes.c_void_p * TTQ_LINEAR_STAGE_EVENTS)()
        for i in range(TTQ_LINEAR_STAGE_EVENTS):
            ev = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = ev

    def stage_ms(self) -> dict:
        """Milliseconds per stage (waits for the last event)."""
        h = _hip()
        if h.hipEventSynchronize(self.handles[-1]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        out = {}
        for i, name in enumerate(LINEAR_STAGES):
            ms = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(ms), self.handles[2 * i], self.handles[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = ms.value
        return out

    def __del__(self):
        try:
            h = _hip()
            for ev in self.handles:
                if ev:
                    h.hipEventDestroy(ev)
        except Exception:
            pass


def linear_state(T: int, K: int, M: int, bits: int, group: int, device="cuda") -> dict:
    """Preallocated tensors for the quantization state ttq_linear can fill."""
    return {
        "ssq": torch.empty(K, dtype=torch.float64, device=device),
        "s": torch.empty(K, dtype=torch.float32, device=device),
        "codes": torch.empty((M, K * bits // 32), dtype=torch.int32, device=device),
        "scale_f16": torch.empty((M, K // group), dtype=torch.float16, device=device),
        "zero_f16": torch.empty((M, K // group), dtype=torch.float16, device=device),
    }
