"""CPU oracle for the TTQ per-prompt hot path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
calls it, and it shares no code with that path: no kernels, helpers, tables or
constants.  Inputs come from the seeded generators (numpy arrays; bf16 as
uint16 bit patterns), decoded here by this module's own code.

Source of the method
--------------------
All citations refer to the nubint.ai review page "[논문 리뷰] TTQ:
Activation-Aware Test-Time Quantization to Accelerate LLM Inference On The
Fly" (Koike-Akino, Liu et al., arXiv 2026), section "제안 방법" (proposed
method), bullets b1..b7, and section "주요 결과" (key results), bullets r1..r5.
Short form used below: [TTQ §method b3].

  b1  weights are quantized on the fly by group-wise RTN with QDQ operations
  b2  AWQ with a diagonal approximation of the input covariance gives a fast
      closed form
  b3  activation statistics are estimated online during inference, and a
      shrunk C_lambda is used to minimise L = E_X ||(W - W_hat) X||^2
  b4  alpha, lambda and p are fixed in advance (no search at test time)
  b5  optional dynamic low-rank factors: W = W_q + B A, W_q quantized at once
  b7  a quantized projection kernel runs the quantized layer on the GPU

Readings where the page is silent (each listed in the design notes):
  * diagonal covariance = uncentered per-channel mean of squares over the
    prompt's tokens (the loss in b3 expands with E[X X^T]);
  * shrinkage = ridge: C + lambda I, lambda = lambda_rel * mean_j(c_j);
  * p = moment order of the per-channel magnitude: c_j = mean_t |x_tj|^p
    (p = 2: the diagonal covariance; p = 1: mean |x|, AWQ's own statistic),
    s_j = (c_j + lambda)^(alpha/p); s_j = 1 where c_j + lambda == 0;
  * group = g consecutive input channels of one output row;
  * asymmetric RTN with a 0-extended range and an integer zero point;
    the step is stored as fp16 rounded toward +inf (so the grid covers the
    range); ties round to even; a NaN value gets code 0;
  * codes form a little-endian bit stream per row (code j in bits
    [b*j, b*j + b)), 32-bit words;
  * low-rank residual accumulated in fp64 in rank order, then scaled by s
    in fp64 and rounded once more to fp32;
  * low-rank factors: top-r SVD of W diag(s); B = U_r S_r, A = V_r^T diag(1/s).

Floating-point conventions: fp64 everywhere, except where a stored precision
is part of the definition (the fp32 value to quantize, the fp32 step
arithmetic, the fp16 step/zero and the fp32 code decision).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode", "stats", "awq_scales", "quant_values", "group_rtn", "pack_codes",
    "unpack_codes", "dequant", "effective_weight", "project", "loss",
    "lowrank_factors", "lowrank_factors_randomized", "linear", "boundary_band",
]


# ------------------------------------------------------------------ inputs

def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Input array -> exact fp64 values.  bf16 arrives as uint16 bit patterns:
    a bf16 value is the fp32 value whose upper 16 bits are those bits."""
    if dtype == "bf16":
        bits32 = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------- statistics

def stats(X: np.ndarray, xdtype: str, ssq_prev: np.ndarray | None = None,
          p: float = 2.0) -> np.ndarray:
    """Per-channel sum of |x|^p of the prompt activations, fp64.

    [TTQ §method b2, b3]: the activation statistics that the closed form uses
    are the diagonal of the input covariance; here ssq_j = sum_t x_tj^2 (the
    division by the token count happens in `awq_scales`).  [TTQ §method b4]
    fixes p in advance; for p != 2 the statistic is the p-th absolute moment
    sum, sum_t |x_tj|^p (p arrives as an fp32 number, widened exactly).
    ``ssq_prev`` adds the sums of earlier chunks of the same prompt.
    """
    x = decode(X, xdtype)
    pp = float(np.float32(p))
    if pp == 2.0:
        m = x * x
    elif pp == 1.0:
        m = np.abs(x)
    else:
        m = np.power(np.abs(x), pp)
    ssq = np.sum(m, axis=0, dtype=np.float64)
    if ssq_prev is not None:
        ssq = np.asarray(ssq_prev, dtype=np.float64) + ssq
    return ssq


def awq_scales(ssq: np.ndarray, n_tokens: int, alpha: float, lambda_rel: float,
               p: float = 2.0) -> np.ndarray:
    """Shrunk AWQ per-channel scales, fp32.

    [TTQ §method b2-b4]: c_j = ssq_j / T is the diagonal covariance estimate;
    the shrunk estimate is c_j + lambda with lambda = lambda_rel * mean(c);
    the AWQ scale is the channel magnitude raised to the fixed alpha, here
    s_j = (c_j + lambda)^(alpha/p), where ssq holds the p-th moment sums of
    `stats` with the same p (p = 2: sums of squares), evaluated in fp64 and
    rounded once to fp32.  alpha, lambda_rel and p arrive as fp32 numbers and
    are widened exactly.  Where c_j + lambda == 0 the scale is defined as 1.
    """
    if not (np.isfinite(np.float32(p)) and float(np.float32(p)) > 0.0):
        raise ValueError("p must be finite and > 0")
    ssq = np.asarray(ssq, dtype=np.float64)
    K = ssq.shape[0]
    c = ssq / np.float64(n_tokens)
    lam = np.float64(np.float32(lambda_rel)) * (np.sum(c) / np.float64(K))
    cl = c + lam
    e = np.float64(np.float32(alpha)) / np.float64(np.float32(p))
    s64 = np.power(cl, e)
    s64 = np.where(cl == 0.0, 1.0, s64)
    return s64.astype(np.float32)


# -------------------------------------------------------------- quantizer

def quant_values(W: np.ndarray, wdtype: str, s: np.ndarray,
                 B: np.ndarray | None = None, A: np.ndarray | None = None) -> np.ndarray:
    """The fp32 values that get quantized: (W - B A) diag(s).

    [TTQ §method b2] AWQ quantizes the weight scaled per input channel by s;
    [TTQ §method b5] with low-rank factors it is the residual W - B A that is
    quantized.  acc starts at W (exact in fp64); each rank k subtracts the
    fp64 product B_ok * A_kj (exact: both are fp32); then acc * s_j is formed
    in fp64 and rounded to fp32.  Without factors this is the correctly
    rounded fp32 product W_oj * s_j.
    """
    acc = decode(W, wdtype).copy()
    if B is not None:
        B64 = np.asarray(B, dtype=np.float32).astype(np.float64)
        A64 = np.asarray(A, dtype=np.float32).astype(np.float64)
        for k in range(B64.shape[1]):
            acc -= np.outer(B64[:, k], A64[k, :])
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    return (acc * s64[None, :]).astype(np.float32)


def _fp16_round_up(d32: np.ndarray) -> np.ndarray:
    """fp32 -> fp16, rounded toward +infinity."""
    h = d32.astype(np.float16)                       # nearest-even first
    low = h.astype(np.float32) < d32
    h[low] = np.nextafter(h[low], np.float16(np.inf))
    return h


def group_rtn(v: np.ndarray, bits: int, group: int) -> dict:
    """Group-wise asymmetric round-to-nearest quantization.

    [TTQ §method b1]: each group of ``group`` consecutive input channels of
    one output row gets its own step and zero point.  For a group:
      mn = min(0, min v), mx = max(0, max v)           (NaNs ignored)
      d32 = fp32(mx - mn) / (2^b - 1)                  (fp32 arithmetic)
      delta = fp16(d32) rounded up; delta = 1 if d32 == 0
      z = clamp(rne(fp32(-mn / delta)), 0, 2^b - 1)
      u = fp32(v / delta)                              (the pre-rounding value)
      q = clamp(rne(u) + z, 0, 2^b - 1); q = 0 where v is NaN
    Returns q (int64 [M][K]), delta and zero (fp16 [M][K/g]) and u.
    """
    v = np.asarray(v, dtype=np.float32)
    M, K = v.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    qmax = np.float32(2 ** bits - 1)
    vg = v.reshape(M, K // group, group)
    mn = np.fmin(np.float32(0.0), np.fmin.reduce(vg, axis=2))
    mx = np.fmax(np.float32(0.0), np.fmax.reduce(vg, axis=2))
    d32 = (mx - mn) / qmax
    delta = _fp16_round_up(d32)
    delta[d32 == 0] = np.float16(1.0)
    df = delta.astype(np.float32)
    zero = np.clip(np.rint((-mn) / df), np.float32(0.0), qmax)
    u = vg / df[:, :, None]
    with np.errstate(invalid="ignore"):
        qf = np.clip(np.rint(u) + zero[:, :, None], np.float32(0.0), qmax)
    qf = np.where(np.isnan(u), np.float32(0.0), qf)
    return {
        "q": qf.reshape(M, K).astype(np.int64),
        "delta": delta,
        "zero": zero.astype(np.float16),
        "u": u.reshape(M, K),
    }


def boundary_band(u: np.ndarray, tol: float = 1e-4) -> np.ndarray:
    """Elements whose pre-rounding value lies within ``tol`` of a step of a
    rounding boundary (a half-integer): there, two codes are acceptable."""
    u = np.asarray(u, dtype=np.float64)
    frac = u - np.floor(u)
    return np.abs(frac - 0.5) < tol


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack each row's codes as a little-endian bit stream of int32 words.

    Code j of a row occupies stream bits [b*j, b*j + b), its least
    significant bit first; stream bit i is bit (i mod 32) of word i // 32.
    """
    q = np.asarray(q, dtype=np.int64)
    M, K = q.shape
    if (K * bits) % 32:
        raise ValueError("K * bits must be a multiple of 32")
    nwords = K * bits // 32
    out = np.empty((M, nwords), dtype=np.uint32)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    step = max(1, (1 << 22) // max(1, K * bits))
    for r0 in range(0, M, step):
        qr = q[r0:r0 + step].astype(np.uint64)
        stream = np.empty((qr.shape[0], K * bits), dtype=np.uint64)
        for i in range(bits):
            stream[:, i::bits] = (qr >> np.uint64(i)) & np.uint64(1)
        out[r0:r0 + step] = (stream.reshape(qr.shape[0], nwords, 32) * weights).sum(axis=2)
    return out.view(np.int32)


def unpack_codes(codes: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of `pack_codes`."""
    words = np.asarray(codes).view(np.uint32).astype(np.uint64)
    M = words.shape[0]
    shifts = np.arange(32, dtype=np.uint64)
    stream = ((words[:, :, None] >> shifts) & np.uint64(1)).reshape(M, -1)[:, :K * bits]
    q = np.zeros((M, K), dtype=np.int64)
    for i in range(bits):
        q |= stream[:, i::bits].astype(np.int64) << i
    return q


def dequant(q: np.ndarray, delta: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """QDQ's dequantize half [TTQ §method b1]: w_hat = (q - z) * delta, fp64
    (exact: small integers times an fp16 value)."""
    M, K = q.shape
    d = np.repeat(np.asarray(delta, dtype=np.float64), group, axis=1)
    z = np.repeat(np.asarray(zero, dtype=np.float64), group, axis=1)
    return (np.asarray(q, dtype=np.float64) - z) * d


def effective_weight(w_hat: np.ndarray, s: np.ndarray,
                     B: np.ndarray | None = None, A: np.ndarray | None = None) -> np.ndarray:
    """The weight the quantized layer applies in the original domain:
    W_eff = w_hat diag(1/s) (+ B A) [TTQ §method b2, b5]."""
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    w = w_hat / s64[None, :]
    if B is not None:
        w = w + np.asarray(B, np.float32).astype(np.float64) @ np.asarray(A, np.float32).astype(np.float64)
    return w


# ---------------------------------------------------------------- projection

def project(X: np.ndarray, xdtype: str, s: np.ndarray, w_hat: np.ndarray,
            B: np.ndarray | None = None, A: np.ndarray | None = None) -> np.ndarray:
    """The quantized projection, fp64, Y [T][M].

    [TTQ §method b2, b7]: Y_to = sum_j w_hat_oj * (x_tj / s_j); with the
    low-rank factors of [TTQ §method b5] it adds sum_k B_ok (sum_j A_kj x_tj).
    ``w_hat`` may hold a subset of the output rows (then Y has those columns).
    """
    x = decode(X, xdtype)
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    y = (x / s64[None, :]) @ np.asarray(w_hat, dtype=np.float64).T
    if B is not None:
        A64 = np.asarray(A, np.float32).astype(np.float64)
        B64 = np.asarray(B, np.float32).astype(np.float64)
        y = y + (x @ A64.T) @ B64.T
    return y


def loss(X: np.ndarray, xdtype: str, W: np.ndarray, wdtype: str, w_eff: np.ndarray) -> float:
    """[TTQ §method b3]: L = ||(W - W_eff) X||_F^2 over the prompt's tokens
    (the expectation over X taken as the sum over the T tokens)."""
    x = decode(X, xdtype)
    dw = decode(W, wdtype) - w_eff
    r = x @ dw.T
    return float(np.sum(r * r))


def lowrank_factors(W: np.ndarray, wdtype: str, s: np.ndarray, rank: int):
    """Dynamic low-rank factors [TTQ §method b5], reading: the top-``rank``
    SVD of W diag(s), B = U_r S_r and A = V_r^T diag(1/s), both rounded to
    fp32, so that B A approximates W and B (A X) acts on the raw input."""
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    ws = decode(W, wdtype) * s64[None, :]
    U, S, Vt = np.linalg.svd(ws, full_matrices=False)
    B = (U[:, :rank] * S[None, :rank]).astype(np.float32)
    A = (Vt[:rank, :] / s64[None, :]).astype(np.float32)
    return B, A


def _orth(Y: np.ndarray) -> np.ndarray:
    """Orthonormal basis of range(Y): the Q of Y = Q R with diag(R) > 0 (the
    unique thin QR of a full-column-rank Y), via numpy's Householder QR."""
    Q, R = np.linalg.qr(Y)
    d = np.sign(np.diag(R))
    d[d == 0] = 1.0
    return Q * d[None, :]


def lowrank_factors_randomized(W: np.ndarray, wdtype: str, s: np.ndarray, rank: int,
                               omega: np.ndarray, q: int):
    """Dynamic low-rank factors computed per prompt [TTQ §method b5: the
    factors are dynamic].  Reading: the top-``rank`` factors of W diag(s)
    estimated by randomized subspace iteration (Halko, Martinsson and Tropp,
    "Finding structure with randomness", 2011: the range finder with q power
    iterations, then the SVD of the small projected matrix).

    ``omega`` is the l x K Gaussian test matrix (l >= rank), one test vector
    per row, drawn by the caller.  With A_s = W diag(s):
      Q = orth(A_s omega^T); q times: Q = orth(A_s orth(A_s^T Q));
      C = Q^T A_s (l x K) = U~ S V^T;  U = Q U~;
      B = U_r S_r, A = V_r^T diag(1/s), rounded to fp32 (as `lowrank_factors`).
    fp64 throughout; orth is the Q of a thin QR with a positive diagonal.
    """
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    As = decode(W, wdtype) * s64[None, :]
    Om = np.asarray(omega, dtype=np.float32).astype(np.float64)
    Q = _orth(As @ Om.T)
    for _ in range(q):
        Z = _orth(As.T @ Q)
        Q = _orth(As @ Z)
    C = Q.T @ As
    Ut, S, Vt = np.linalg.svd(C, full_matrices=False)
    U = Q @ Ut
    B = (U[:, :rank] * S[None, :rank]).astype(np.float32)
    A = (Vt[:rank, :] / s64[None, :]).astype(np.float32)
    return B, A


# ------------------------------------------------------------------ composite

def linear(X, xdtype, W, wdtype, bits, group, alpha, lambda_rel, p=2.0,
           B=None, A=None, rows=None) -> dict:
    """The whole per-prompt path for one linear layer [TTQ §method b1-b5]:
    stats -> shrunk AWQ scales -> values -> group RTN -> pack -> projection.
    ``rows`` restricts the quantization and the projection to a subset of
    output rows (for sampled checks at full size)."""
    T = np.asarray(X).shape[0]
    ssq = stats(X, xdtype, p=p)
    s = awq_scales(ssq, T, alpha, lambda_rel, p)
    Wr = W if rows is None else np.asarray(W)[rows]
    Br = None if B is None else (B if rows is None else np.asarray(B)[rows])
    v = quant_values(Wr, wdtype, s, Br, A)
    qr = group_rtn(v, bits, group)
    w_hat = dequant(qr["q"], qr["delta"], qr["zero"], group)
    Y = project(X, xdtype, s, w_hat, Br, A)
    return {"ssq": ssq, "s": s, "v": v, "q": qr["q"], "delta": qr["delta"],
            "zero": qr["zero"], "u": qr["u"], "codes": pack_codes(qr["q"], bits),
            "w_hat": w_hat, "Y": Y}
