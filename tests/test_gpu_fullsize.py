"""Parity at the five benchmark workloads' full sizes.

The layer runs through ttq_linear in the configuration bench.py times: fp32
Y, the prompt state returned, one workspace.  The checks are:

- the statistics and scales of all K channels;
- the quantization of sampled output rows against the oracle's own, using
  the same bars as tests/test_gpu_parity.py;
- Y on those rows for every token;
- Y on every output for sampled tokens, against the dense projection of the
  library's own quantized state (which covers every output tile);
- for the 14336->4096 workload, the decode steps (T = 1, 4, 16) on the prompt
  state.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import host, rel_fro, say, to_dev, f32_dev
from online_activation_aware_amd import synth

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
S_TOL = 1e-5
N_ROWS = 64
N_TOKENS = 24


@pytest.fixture(scope="module")
def T():
    from online_activation_aware_amd import ttq
    ttq.lib()
    return ttq


def _sample(n, k, seed, must=()):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(n, min(k, n), replace=False).tolist()) | {i for i in must if 0 <= i < n}
    return np.array(sorted(pick))


def _run(T, wl, d, B, A):
    X = to_dev(d["X"], wl.xdtype)
    W = to_dev(d["W"], wl.wdtype)
    st = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
    ws = T.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group, wl.rank)
    Y = torch.empty((wl.T, wl.M), dtype=torch.float32, device="cuda")
    T.ttq_linear(X, W, wl.bits, wl.group, wl.alpha, wl.lambda_rel,
                 B=None if B is None else f32_dev(B), A=None if A is None else f32_dev(A),
                 Y=Y, ws=ws, state=st)
    torch.cuda.synchronize()
    return Y, st


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_fullsize_linear(T, key):
    wl = synth.workload(key)
    say(f"full size {key}: {wl.name}")
    d = synth.make_inputs(wl)
    B = A = None
    if wl.rank:
        s0 = oracle.awq_scales(oracle.stats(d["X"], wl.xdtype), wl.T, wl.alpha, wl.lambda_rel)
        B, A = oracle.lowrank_factors(d["W"], wl.wdtype, s0, wl.rank)
    rows = _sample(wl.M, N_ROWS, 11, must=(0, wl.M - 1))
    ref = oracle.linear(d["X"], wl.xdtype, d["W"], wl.wdtype, wl.bits, wl.group, wl.alpha,
                        wl.lambda_rel, B=B, A=A, rows=rows)
    Y, st = _run(T, wl, d, B, A)

    # statistics and scales: every channel
    np.testing.assert_allclose(host(st["ssq"]), ref["ssq"], rtol=1e-12)
    s = host(st["s"])
    np.testing.assert_allclose(s, ref["s"], rtol=S_TOL)
    say(f"  scales identical: {np.array_equal(s, ref['s'])}")

    # quantization of the sampled rows
    codes, delta, zero = host(st["codes"])[rows], host(st["scale_f16"])[rows], host(st["zero_f16"])[rows]
    if np.array_equal(s, ref["s"]):
        np.testing.assert_array_equal(delta.view(np.float16), ref["delta"])
        np.testing.assert_array_equal(zero.view(np.float16), ref["zero"])
        gq = oracle.unpack_codes(codes, wl.bits, wl.K)
        bad = (gq != ref["q"]) & ~oracle.boundary_band(ref["u"])
        assert not bad.any(), f"{int(bad.sum())} codes differ outside the rounding band"

    # Y on the sampled rows, every token, against the oracle's own quantization
    Yh = host(Y)
    err = rel_fro(Yh[:, rows], ref["Y"])
    say(f"  Y rel err (sampled rows, all tokens) {err:.3e}")
    assert err < Y_TOL

    # Y on every output for sampled tokens, against the library's own state
    toks = _sample(wl.T, N_TOKENS, 12, must=(0, wl.T - 1))
    gq_all = oracle.unpack_codes(host(st["codes"]), wl.bits, wl.K)
    w_hat = oracle.dequant(gq_all, host(st["scale_f16"]).view(np.float16),
                           host(st["zero_f16"]).view(np.float16), wl.group)
    Xs = np.asarray(d["X"])[toks]
    ref_all = oracle.project(Xs, wl.xdtype, s, w_hat, B, A)
    err_all = rel_fro(Yh[toks], ref_all)
    say(f"  Y rel err (all outputs, sampled tokens) {err_all:.3e}")
    assert err_all < Y_TOL
    col_err = np.linalg.norm(Yh[toks] - ref_all, axis=0) / np.maximum(np.linalg.norm(ref_all, axis=0), 1e-30)
    assert np.all(col_err < 2e-2), f"worst output column {int(np.argmax(col_err))}: {col_err.max():.3e}"

    if wl.decode_T:
        ws = T.workspace(max(wl.decode_T), wl.K, wl.M, wl.bits, wl.group)
        for td, Xd in d["X_decode"].items():
            Yd = T.ttq_qgemm(to_dev(Xd, wl.xdtype), st["s"], st["codes"], st["scale_f16"], st["zero_f16"],
                             wl.M, wl.bits, wl.group, ws=ws)
            Ydh = host(Yd)
            e1 = rel_fro(Ydh[:, rows], oracle.project(Xd, wl.xdtype, ref["s"], ref["w_hat"]))
            e2 = rel_fro(Ydh, oracle.project(Xd, wl.xdtype, s, w_hat))
            say(f"  decode T={td}: rel err {e1:.3e} (oracle rows), {e2:.3e} (all outputs)")
            assert e1 < Y_TOL and e2 < Y_TOL
