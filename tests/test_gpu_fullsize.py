"""Parity at the five benchmark workloads' full sizes.

The layer runs through ttq_linear in the configuration bench.py times: fp32
Y, the prompt state returned, one workspace.  The checks are:

- the statistics and scales of all K channels (scales bit-identical to the
  oracle's in almost every channel);
- the quantization of sampled output rows against the oracle's group RTN on
  the library's own scales (steps and zeros exact, codes exact outside the
  rounding band, at most 1e-4 of them inside it);
- Y on those rows for every token against the oracle (relative Frobenius);
- every element of Y against the fp64 projection of the library's own
  quantized state, within the element-wise bound of the single bf16 rounding
  of the dequantized weight (tests/gpu_util.py);
- for the 14336->4096 workload, the decode steps (T = 1, 4, 16) on the prompt
  state, the same way.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (check_quant_state, check_scales, f32_dev, host, rel_fro, say, to_dev,
                      y_elementwise_check)
from online_activation_aware_amd import synth

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
S_TOL = 1e-5
N_ROWS = 64


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
    check_scales(s, ref["s"], rtol=S_TOL)
    say(f"  scales identical: {np.array_equal(s, ref['s'])}")

    # quantization of the sampled rows, against the oracle on the library's s
    codes_all, delta_all, zero_all = host(st["codes"]), host(st["scale_f16"]), host(st["zero_f16"])
    nb = check_quant_state(codes_all[rows], delta_all[rows], zero_all[rows], np.asarray(d["W"])[rows],
                           wl.wdtype, s, wl.bits, wl.group, None if B is None else B[rows], A)
    say(f"  quantizer: {nb} in-band code differences on {len(rows)} rows")

    # Y on the sampled rows, every token, against the oracle's own quantization
    Yh = host(Y)
    err = rel_fro(Yh[:, rows], ref["Y"])
    say(f"  Y rel err (sampled rows, all tokens) {err:.3e}")
    assert err < Y_TOL

    # every element of Y against the fp64 projection of the library's state
    q_all = oracle.unpack_codes(codes_all, wl.bits, wl.K)
    d16, z16 = delta_all.view(np.float16), zero_all.view(np.float16)
    worst = y_elementwise_check(Yh, d["X"], wl.xdtype, s, q_all, d16, z16, wl.group, B, A)
    say(f"  Y element-wise: worst |error| / bound {worst:.3f}")

    if not wl.rank and wl.xdtype == "bf16" and wl.M * wl.K * 2 > 64 << 20:
        # The prompt projected again from the stored state through ttq_qgemm:
        # its dequantize kernel writes w~ with streaming stores at this size
        # (like the quantizer inside ttq_linear), with the same arithmetic, and
        # the same GEMM runs, so Y must be bitwise the same.
        ws_p = T.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group)
        Yq = T.ttq_qgemm(to_dev(d["X"], wl.xdtype), st["s"], st["codes"], st["scale_f16"], st["zero_f16"],
                         wl.M, wl.bits, wl.group, ws=ws_p)
        torch.cuda.synchronize()
        assert np.array_equal(host(Yq), Yh), "ttq_qgemm on the stored state differs from ttq_linear"
        say("  ttq_qgemm on the stored state: bitwise equal to ttq_linear")
        del Yq, ws_p

    if wl.decode_T:
        ws = T.workspace(max(wl.decode_T), wl.K, wl.M, wl.bits, wl.group)
        for td, Xd in d["X_decode"].items():
            Yd = T.ttq_qgemm(to_dev(Xd, wl.xdtype), st["s"], st["codes"], st["scale_f16"], st["zero_f16"],
                             wl.M, wl.bits, wl.group, ws=ws)
            Ydh = host(Yd)
            e1 = rel_fro(Ydh[:, rows], oracle.project(Xd, wl.xdtype, ref["s"], ref["w_hat"]))
            wd = y_elementwise_check(Ydh, Xd, wl.xdtype, s, q_all, d16, z16, wl.group,
                                     valu=(td <= 4 and wl.K % 128 == 0))
            say(f"  decode T={td}: rel err {e1:.3e} (oracle rows), element-wise worst ratio {wd:.3f}")
            assert e1 < Y_TOL
