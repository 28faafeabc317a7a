"""Helpers for the GPU parity tests: move the generators' numpy arrays to the
device as exactly the same bytes, and read results back."""
import sys

import numpy as np
import torch


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Encoded host array (fp32, or bf16 as uint16 bits) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to("cuda")


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def f16_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float16))).to("cuda")


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


# ------------------------------------------------------------ parity checks
#
# Codes: bit-exact wherever the oracle's pre-rounding value v / step lies more
# than 1e-4 of a step from a rounding boundary; inside that band either
# neighbouring code is accepted.  Two kinds of values lie in the band:
# - exact ties, v / step = k + 1/2 exactly (common when v has few significant
#   bits, e.g. bf16 weights with s = 1): the oracle rounds them to even, the
#   library decides on v * (1/step), which puts a tie on either side;
# - near-ties: there the library's v * (1/step), a few ulps from v / step,
#   agrees with the oracle except within ~1e-6 of the boundary, so such
#   differences must stay rare: at most 1e-4 of all codes.
MAX_BAND_MISMATCH_FRAC = 1e-4


def exact_ties(v, delta, group):
    """Mask of the values whose quotient v / step is exactly k + 1/2 (fp64:
    the quotient of an fp32 value by an fp16 step is checked by multiplying
    back, exact in fp64)."""
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    d64 = np.repeat(np.asarray(delta, dtype=np.float16).astype(np.float64), group, axis=1)
    with np.errstate(invalid="ignore"):
        t = v64 / d64
        return ((t - np.floor(t)) == 0.5) & (t * d64 == v64)


def check_codes(got_codes, or_q, or_u, bits, K, ties=None):
    """Packed GPU codes against the oracle's codes; returns the number of
    in-band differences.  Differences outside the band fail; in-band ones
    other than exact ties (``ties``, a mask) must be at most 1e-4 of all
    codes."""
    import oracle
    gq = oracle.unpack_codes(got_codes, bits, K)
    band = oracle.boundary_band(or_u)
    diff = gq != or_q
    bad = diff & ~band
    assert not bad.any(), f"{int(bad.sum())} codes differ outside the rounding band"
    near = diff & band if ties is None else diff & band & ~np.asarray(ties)
    n_near = int(near.sum())
    assert n_near <= MAX_BAND_MISMATCH_FRAC * gq.size, \
        f"{n_near} in-band code differences (not exact ties) out of {gq.size}"
    if ties is not None:   # a tie's code is one of its two neighbours
        t = np.asarray(ties) & diff
        assert np.all(np.abs(gq[t] - or_q[t]) == 1)
    # the GPU's words are a valid packing of its codes (layout round trip)
    np.testing.assert_array_equal(oracle.pack_codes(gq, bits), got_codes)
    return int((diff & band).sum())


def check_quant_state(codes, scale_f16, zero_f16, W, wdtype, s, bits, group, B=None, A=None):
    """The library's quantized state (host arrays) against the oracle's group
    RTN of (W - B A) diag(s), where s is the scale vector the library itself
    used: steps and zeros exact, codes as in check_codes."""
    import oracle
    K = np.asarray(W).shape[1]
    v = oracle.quant_values(W, wdtype, s, B, A)
    r = oracle.group_rtn(v, bits, group)
    np.testing.assert_array_equal(np.asarray(scale_f16).view(np.float16), r["delta"])
    np.testing.assert_array_equal(np.asarray(zero_f16).view(np.float16), r["zero"])
    return check_codes(codes, r["q"], r["u"], bits, K, exact_ties(v, r["delta"], group))


def check_scales(s_gpu, s_ref, rtol=1e-5, min_equal=0.999):
    """Scales within rtol, and bit-identical in almost every channel (both
    sides evaluate the same fp64 power and round once to fp32; only a one-ulp
    difference of the fp64 pow next to an fp32 rounding boundary can differ)."""
    np.testing.assert_allclose(s_gpu, s_ref, rtol=rtol)
    eq = float(np.mean(np.asarray(s_gpu) == np.asarray(s_ref)))
    assert eq >= min_equal, f"only {eq:.5f} of the scales are bit-identical"


def y_elementwise_check(got, X, xdtype, s, q, delta, zero, group, B=None, A=None, valu=False,
                        y_bf16=False, rows=None):
    """Every element of Y against the fp64 projection of the given quantized
    state (q [M'][K] codes, steps, zeros), within a bound derived from the
    library's arithmetic:

    - matrix-core paths: the dequantized weight (q - z) step (1/s) is rounded
      once to bf16 (relative error <= 2^-8; fp32 X splits X and the weight
      into two bf16 halves each: <= 2^-14), products accumulated in fp32;
    - the few-token vector path (valu=True): fp32 throughout, the group map
      applied to sums, so errors scale with step (q + z) / s rather than with
      the dequantized weight;
    - fp32 accumulation over K terms: K 2^-23 relative to the sum of the
      absolute products (a worst-case bound, twice the textbook gamma_K;
      three times that for the three products of split fp32 X);
    - the low-rank term B (A X) in fp32: (K + rank + 4) 2^-23 relative to
      sum_k |B_ok| sum_j |A_kj x_tj|;
    - a bf16 Y adds 2^-8 |Y|.
    rows: the output rows (columns of Y) that q, delta, zero and B hold.
    Returns the largest ratio |error| / bound."""
    import oracle
    x = oracle.decode(X, xdtype)
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    w_hat = oracle.dequant(q, delta, zero, group)
    K = x.shape[1]
    ref = oracle.project(X, xdtype, s, w_hat, B, A)
    if valu:
        d = np.repeat(np.asarray(delta, np.float64), group, axis=1)
        z = np.repeat(np.asarray(zero, np.float64), group, axis=1)
        mag = d * (np.asarray(q, np.float64) + z) / s64[None, :]
        rel = 2.0 ** -21
    else:
        mag = np.abs(w_hat) / s64[None, :]
        rel = 2.0 ** -8 if xdtype == "bf16" else 2.0 ** -14
    ax = np.abs(x)
    nprod = 3 if (xdtype == "f32" and not valu) else 1
    bound = (ax @ mag.T) * (rel + nprod * K * 2.0 ** -23)
    if B is not None:
        B64 = np.abs(np.asarray(B, np.float32).astype(np.float64))
        A64 = np.abs(np.asarray(A, np.float32).astype(np.float64))
        bound += ((ax @ A64.T) @ B64.T) * ((K + B64.shape[1] + 4) * 2.0 ** -23)
    bound += np.abs(ref) * (2.0 ** -8 if y_bf16 else 2.0 ** -22) + 1e-30
    g = np.asarray(got, dtype=np.float64)
    if rows is not None:
        g = g[:, rows]
    err = np.abs(g - ref)
    worst = float(np.max(err / bound))
    assert np.all(np.isfinite(g)), "non-finite outputs"
    assert worst <= 1.0, (f"{int((err > bound).sum())} outputs outside the element-wise bound "
                          f"(worst ratio {worst:.3f} at {np.unravel_index(np.argmax(err / bound), err.shape)})")
    return worst
