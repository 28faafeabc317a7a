"""Seeded synthetic inputs for the TTQ layer workloads.

This module only draws random numbers and encodes them as fp32 or bf16 bytes.
It holds none of the quantization method's arithmetic, so both the CPU oracle
(through the tests) and the HIP path receive the very same input bytes from
it.

The workloads stand in for the layers the TTQ review page evaluates on
(OPT-125M up to Gemma-1B, Qwen3; "Key results" section): the public
perplexity datasets and trained weights are not used.  Shapes are the
models' projection shapes; activations carry heavy outlier channels the way
LLM activations do.

bf16 tensors are returned as ``np.uint16`` bit patterns (numpy has no bf16).

Recipe (per workload ``i``): ``SeedSequence(1000 + i).spawn(5)`` gives five
independent streams, for X, W, the outlier channel indices, the planted
low-rank factors and the decode tokens.  Everything is drawn in fp64 and
rounded once, to fp32 (RNE) or to bf16 (fp64 -> fp32 -> bf16, RNE each).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic linear layer: sizes, dtypes, quantizer settings."""

    key: str            # c1 .. c5
    name: str           # descriptive workload name
    T: int              # prompt tokens
    K: int              # input channels (d)
    M: int              # output channels (d')
    xdtype: str         # "f32" or "bf16"
    wdtype: str         # "f32" or "bf16"
    bits: int
    group: int
    alpha: float = 0.5
    lambda_rel: float = 1e-2
    rank: int = 0
    x_law: str = "normal_outliers"   # or "student_t_lognormal"
    n_outliers: Optional[int] = None  # None -> round(0.01 K)
    outlier_factor: float = 30.0
    w_sigma: float = 0.015
    planted_norm: float = 0.0        # spectral norm of the planted rank-r part
    decode_T: tuple = field(default_factory=tuple)
    index: int = 0


WORKLOADS = {
    "c1": Workload("c1", "opt125m_qproj_768x768_t128_fp32", 128, 768, 768, "f32", "f32",
                   4, 32, n_outliers=8, outlier_factor=20.0, w_sigma=0.02, index=1),
    "c2": Workload("c2", "attn_proj_4096x4096_t2048_bf16_b4g32", 2048, 4096, 4096, "bf16", "bf16",
                   4, 32, w_sigma=0.015, index=2),
    "c3": Workload("c3", "mlp_up_4096x14336_t512_bf16_b3g16", 512, 4096, 14336, "bf16", "bf16",
                   3, 16, x_law="student_t_lognormal", w_sigma=0.01, index=3),
    "c4": Workload("c4", "mlp_down_14336x4096_prefill1024_decode_bf16_b4g32", 1024, 14336, 4096,
                   "bf16", "bf16", 4, 32, w_sigma=0.01, decode_T=(1, 4, 16), index=4),
    "c5": Workload("c5", "lowrank_4096x4096_t2048_bf16_b2g32_r16", 2048, 4096, 4096, "bf16", "bf16",
                   2, 32, rank=16, w_sigma=0.015, planted_norm=5.0, index=5),
}


def workload(key: str, **overrides) -> Workload:
    """The named workload, optionally with other sizes (same value laws)."""
    return replace(WORKLOADS[key], **overrides)


# ----------------------------------------------------------------- encoding

def f64_to_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(f64_to_f32(a))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (used for display/inputs)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return f64_to_f32(a64)
    if dtype == "bf16":
        return f64_to_bf16_bits(a64)
    raise ValueError(dtype)


# --------------------------------------------------------------- generators

def _streams(wl: Workload, seed: Optional[int]):
    base = 1000 + wl.index if seed is None else seed
    return [np.random.default_rng(s) for s in np.random.SeedSequence(base).spawn(5)]


def _outlier_channels(rng, K: int, n: int) -> np.ndarray:
    n = max(0, min(K, n))
    return np.sort(rng.choice(K, n, replace=False))


def _draw_x(wl: Workload, rng_x, chans, sig, T: int) -> np.ndarray:
    if wl.x_law == "normal_outliers":
        x = rng_x.standard_normal((T, wl.K))
        x[:, chans] *= wl.outlier_factor
    elif wl.x_law == "student_t_lognormal":
        x = rng_x.standard_t(4.0, size=(T, wl.K)) * sig[None, :]
    else:
        raise ValueError(wl.x_law)
    return x


def make_inputs(wl: Workload, seed: Optional[int] = None) -> dict:
    """Draw X [T][K], W [M][K] (and decode tokens) for a workload.

    Returns a dict with the encoded arrays ``X``, ``W``, ``X_decode`` (a dict
    T -> [T][K] array, for workloads with decode steps) and the metadata used.
    """
    rng_x, rng_w, rng_o, rng_p, rng_d = _streams(wl, seed)
    n_out = wl.n_outliers if wl.n_outliers is not None else int(round(0.01 * wl.K))
    chans = _outlier_channels(rng_o, wl.K, n_out)
    sig = rng_o.lognormal(0.0, 1.0, size=wl.K) if wl.x_law == "student_t_lognormal" else None

    x = _draw_x(wl, rng_x, chans, sig, wl.T)
    w = rng_w.standard_normal((wl.M, wl.K)) * wl.w_sigma
    if wl.planted_norm:
        r = max(wl.rank, 1)
        q1, _ = np.linalg.qr(rng_p.standard_normal((wl.M, r)))
        q2, _ = np.linalg.qr(rng_p.standard_normal((wl.K, r)))
        w = w + wl.planted_norm * (q1 @ q2.T)

    out = {
        "workload": wl,
        "X": encode(x, wl.xdtype),
        "W": encode(w, wl.wdtype),
        "outlier_channels": chans,
        "X_decode": {},
    }
    for td in wl.decode_T:
        out["X_decode"][td] = encode(_draw_x(wl, rng_d, chans, sig, td), wl.xdtype)
    return out


def test_vectors(l: int, K: int, seed: int = 0) -> np.ndarray:
    """l Gaussian test vectors of length K (rows), fp32: the random input of
    the randomized low-rank factorization, drawn by the caller."""
    rng = np.random.default_rng(np.random.SeedSequence(7000 + seed))
    return rng.standard_normal((l, K)).astype(np.float32)


def as_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Encoded array -> exact fp32 values (bf16 widened)."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)
