"""Parity of the per-prompt low-rank factors (ttq_lowrank_factors) with the
oracle's randomized subspace iteration on the same test vectors.

The passes over W run in fp32 on the matrix cores and the small problems in
fp64, so the factors agree with the fp64 oracle to ~1e-7; the bar is 1e-5
relative Frobenius on B A (the unique part) and, where the singular values
are well separated, on B and A themselves after fixing each pair's sign.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import f32_dev, host, rel_fro, say, to_dev
from online_activation_aware_amd import synth

pytestmark = pytest.mark.gpu

F_TOL = 1e-5


@pytest.fixture(scope="module")
def T():
    from online_activation_aware_amd import ttq
    ttq.lib()
    return ttq


def _spectrum_weight(M, K, r, seed):
    """bf16 W with W diag(s) of a known spectrum: r separated values, a tail."""
    rng = np.random.default_rng(seed)
    n = min(M, K)
    sig = np.concatenate([8.0 * 0.8 ** np.arange(r), 0.6 * 0.97 ** np.arange(n - r)])
    U = np.linalg.qr(rng.standard_normal((M, n)))[0]
    V = np.linalg.qr(rng.standard_normal((K, n)))[0]
    s = (rng.random(K) + 0.5).astype(np.float32)
    W = synth.encode((U * sig[None, :]) @ V.T / s.astype(np.float64)[None, :], "bf16")
    return W, s


def _run(T, W, s, om, rank, q):
    B, A = T.ttq_lowrank_factors(to_dev(W, "bf16"), f32_dev(s), f32_dev(om), rank, q)
    torch.cuda.synchronize()
    return host(B).astype(np.float64), host(A).astype(np.float64)


def _sign_fixed(Bg, Ag, Br, Ar):
    d = np.sign(np.sum(Ag * Ar, axis=1))
    d[d == 0] = 1.0
    return Bg * d[None, :], Ag * d[:, None]


@pytest.mark.parametrize("M,K,l,rank,q", [(300, 256, 12, 6, 2), (203, 288, 10, 4, 1), (512, 1024, 24, 16, 0),
                                          (160, 512, 32, 32, 3), (96, 64, 5, 1, 2)])
def test_factors_match_oracle_separated_spectrum(T, M, K, l, rank, q):
    say(f"factors M={M} K={K} l={l} rank={rank} q={q}")
    W, s = _spectrum_weight(M, K, rank, seed=M + K)
    om = synth.test_vectors(l, K, seed=l)
    Br, Ar = oracle.lowrank_factors_randomized(W, "bf16", s, rank, om, q)
    Bg, Ag = _run(T, W, s, om, rank, q)
    Br, Ar = Br.astype(np.float64), Ar.astype(np.float64)
    e_prod = rel_fro(Bg @ Ag, Br @ Ar)
    Bg, Ag = _sign_fixed(Bg, Ag, Br, Ar)
    say(f"  B A {e_prod:.2e}  B {rel_fro(Bg, Br):.2e}  A {rel_fro(Ag, Ar):.2e}")
    assert e_prod < F_TOL
    if rank < l or q > 0:
        assert rel_fro(Bg, Br) < F_TOL and rel_fro(Ag, Ar) < F_TOL


def test_factors_planted_rank16_workload(T):
    # The low-rank workload's weight (planted rank-16 part) at reduced size,
    # with the scales of its prompt, as the path uses it.
    wl, d = synth.workload("c5", T=256, K=1024, M=768), None
    d = synth.make_inputs(wl)
    s = oracle.awq_scales(oracle.stats(d["X"], "bf16"), wl.T, wl.alpha, wl.lambda_rel)
    om = synth.test_vectors(24, wl.K, seed=5)
    Br, Ar = oracle.lowrank_factors_randomized(d["W"], "bf16", s, 16, om, 2)
    Bg, Ag = _run(T, d["W"], s, om, 16, 2)
    err = rel_fro(Bg @ Ag, Br.astype(np.float64) @ Ar.astype(np.float64))
    say(f"  planted rank 16: B A rel err {err:.2e}")
    assert err < F_TOL


def test_factors_zero_weight_and_determinism(T):
    W = synth.encode(np.zeros((64, 128)), "bf16")
    s = np.ones(128, np.float32)
    om = synth.test_vectors(8, 128, seed=1)
    Bg, Ag = _run(T, W, s, om, 4, 1)
    assert np.all(Bg == 0) and np.all(Ag == 0)
    W, s = _spectrum_weight(200, 256, 5, seed=9)
    om = synth.test_vectors(9, 256, seed=2)
    b1, a1 = _run(T, W, s, om, 5, 2)
    b2, a2 = _run(T, W, s, om, 5, 2)
    assert np.array_equal(b1, b2) and np.array_equal(a1, a2)


def test_factors_feed_the_layer(T):
    # Per-prompt factors from the GPU, then the layer with them: Y against the
    # oracle's layer with the oracle's factors from the same test vectors.
    wl = synth.workload("c5", T=192, K=512, M=256)
    d = synth.make_inputs(wl)
    s = oracle.awq_scales(oracle.stats(d["X"], "bf16"), wl.T, wl.alpha, wl.lambda_rel)
    om = synth.test_vectors(24, wl.K, seed=3)
    Br, Ar = oracle.lowrank_factors_randomized(d["W"], "bf16", s, 16, om, 2)
    ref = oracle.linear(d["X"], "bf16", d["W"], "bf16", wl.bits, wl.group, wl.alpha, wl.lambda_rel, B=Br, A=Ar)
    Bd, Ad = T.ttq_lowrank_factors(to_dev(d["W"], "bf16"), f32_dev(s), f32_dev(om), 16, 2)
    Y = T.ttq_linear(to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16"), wl.bits, wl.group, wl.alpha,
                     wl.lambda_rel, B=Bd, A=Ad)
    err = rel_fro(host(Y), ref["Y"])
    say(f"  layer with GPU factors: Y rel err {err:.2e}")
    assert err < 2e-3


def test_factors_full_size_low_rank_workload(T):
    # 4096 x 4096 with the planted rank-16 part, r = 16, l = 24, q = 2:
    # B A on sampled rows.
    wl = synth.workload("c5")
    d = synth.make_inputs(wl)
    s = oracle.awq_scales(oracle.stats(d["X"], "bf16"), wl.T, wl.alpha, wl.lambda_rel)
    om = synth.test_vectors(24, wl.K, seed=4)
    Br, Ar = oracle.lowrank_factors_randomized(d["W"], "bf16", s, 16, om, 2)
    Bg, Ag = _run(T, d["W"], s, om, 16, 2)
    rows = np.random.default_rng(5).choice(wl.M, 48, replace=False)
    err = rel_fro(Bg[rows] @ Ag, Br[rows].astype(np.float64) @ Ar.astype(np.float64))
    say(f"  full size: B A rel err (48 rows) {err:.2e}")
    assert err < F_TOL
