"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Sizes here span several tiles with ragged tails; tests/test_gpu_fullsize.py
covers the benchmark workloads at full size on sampled outputs.
Bars: fp64 statistics to 1e-12 relative; scales within 1e-5 relative; fp16
steps and zero points exact; codes exact except where the oracle's
pre-rounding value lies within 1e-4 of a step of a rounding boundary; the
layer output Y within 2e-3 relative Frobenius error (fp32 Y).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (bf16_bits_to_f64, check_codes, check_quant_state, check_scales, exact_ties, f16_dev, f32_dev,
                      host, i32_dev, rel_fro, say, to_dev, y_elementwise_check)
from online_activation_aware_amd import synth

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3          # relative Frobenius error of Y (fp32 output)
Y_TOL_BF16_OUT = 4e-3  # bf16 output adds one more bf16 rounding (~1.5e-3 in quadrature)
S_TOL = 1e-5


@pytest.fixture(scope="module")
def T():
    from online_activation_aware_amd import ttq
    ttq.lib()
    return ttq


def _inputs(key, seed=None, **sizes):
    wl = synth.workload(key, **sizes)
    return wl, synth.make_inputs(wl, seed=seed)


def _check_rtn(got_codes, got_delta, got_zero, v, bits, group):
    """The library's codes, steps and zeros against the oracle's group RTN
    of the values v."""
    r = oracle.group_rtn(v, bits, group)
    np.testing.assert_array_equal(host(got_delta), r["delta"])
    np.testing.assert_array_equal(host(got_zero), r["zero"])
    return check_codes(host(got_codes), r["q"], r["u"], bits, np.asarray(v).shape[1],
                       exact_ties(v, r["delta"], group))


# ------------------------------------------------------------------ stats

@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("Tn,K", [(1, 512), (77, 1000), (300, 2056), (1031, 4104), (600, 10304), (5000, 24),
                                  (3, 8), (2048, 4096), (1024, 14336)])
def test_stats_parity(T, xdt, Tn, K):
    say(f"stats xdt={xdt} T={Tn} K={K}")
    rng = np.random.default_rng(Tn + K)
    X = synth.encode(rng.standard_normal((Tn, K)) * rng.lognormal(0, 1, K)[None, :], xdt)
    ref = oracle.stats(X, xdt)
    ws = torch.empty(32 * K * 8 + 256, dtype=torch.uint8, device="cuda")  # <= 32 fp64 partial rows
    ssq = torch.empty(K, dtype=torch.float64, device="cuda")
    T.ttq_stats(to_dev(X, xdt), ssq, ws=ws)
    np.testing.assert_allclose(host(ssq), ref, rtol=1e-12, atol=0)


def test_stats_accumulate_and_strided(T):
    say("stats accumulate + strided rows")
    rng = np.random.default_rng(5)
    K = 768
    X = synth.encode(rng.standard_normal((200, K)), "bf16")
    big = torch.zeros((200, K + 64), dtype=torch.bfloat16, device="cuda")
    big[:, :K] = to_dev(X, "bf16")
    ws = T.workspace(200, K, 32, 4, 32)
    ssq = torch.full((K,), 7.0, dtype=torch.float64, device="cuda")
    T.ttq_stats(big[:120, :K], ssq, accumulate=False, ws=ws)
    T.ttq_stats(big[120:, :K], ssq, accumulate=True, ws=ws)
    ref = oracle.stats(X[120:], "bf16", oracle.stats(X[:120], "bf16"))
    np.testing.assert_allclose(host(ssq), ref, rtol=1e-12)


# ------------------------------------------------------------------ scales

@pytest.mark.parametrize("K", [32, 768, 4096, 14336])
@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0])
def test_scales_parity(T, K, alpha):
    say(f"scales K={K} alpha={alpha}")
    rng = np.random.default_rng(K)
    ssq = rng.lognormal(3, 2, K) * 100
    ssq[::97] = 0.0
    ref = oracle.awq_scales(ssq, 123, alpha, 1e-2)
    s = T.ttq_awq_scales(torch.from_numpy(ssq).to("cuda"), 123, alpha, 1e-2)
    got = host(s)
    np.testing.assert_allclose(got, ref, rtol=S_TOL)
    assert np.mean(got == ref) > 0.99
    if alpha == 0.0:
        np.testing.assert_array_equal(got, np.ones(K, np.float32))


def test_scales_zero_input_is_one(T):
    s = T.ttq_awq_scales(torch.zeros(256, dtype=torch.float64, device="cuda"), 8, 0.5, 1e-2)
    np.testing.assert_array_equal(host(s), np.ones(256, np.float32))


@pytest.mark.parametrize("p", [1.0, 3.0, 0.5])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("Tn", [300, 200])     # 200: the one-kernel statistics path
def test_stats_and_scales_moment_p(T, p, xdt, Tn):
    # [TTQ §method b4] p fixed in advance: sums of |x|^p and s = (c + lambda)^(alpha/p).
    say(f"stats p={p} {xdt} T={Tn}")
    key = "c1" if xdt == "f32" else "c2"
    wl, d = _inputs(key, T=Tn, K=1096)
    X = to_dev(d["X"], xdt)
    ws = torch.empty(32 * 1096 * 8, dtype=torch.uint8, device="cuda")   # 32 fp64 partial rows
    msum = T.ttq_stats_p(X, p, torch.empty(1096, dtype=torch.float64, device="cuda"), ws=ws)
    ref = oracle.stats(d["X"], xdt, p=p)
    np.testing.assert_allclose(host(msum), ref, rtol=1e-12)
    s = T.ttq_awq_scales(msum, Tn, 0.5, 1e-2, p=p)
    np.testing.assert_allclose(host(s), oracle.awq_scales(ref, Tn, 0.5, 1e-2, p=p), rtol=1e-6)
    # ttq_stats is the p = 2 case
    ssq = T.ttq_stats(X, torch.empty(1096, dtype=torch.float64, device="cuda"), ws=ws)
    sq2 = T.ttq_stats_p(X, 2.0, torch.empty(1096, dtype=torch.float64, device="cuda"), ws=ws)
    np.testing.assert_array_equal(host(ssq), host(sq2))


def test_stats_p_rejects_nonpositive(T):
    X = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    m = torch.empty(64, dtype=torch.float64, device="cuda")
    for p in (0.0, -2.0, float("nan")):
        with pytest.raises(T.TTQError) as e:
            T.ttq_stats_p(X, p, m, ws=torch.empty(32 * 64 * 8, dtype=torch.uint8, device="cuda"))
        assert e.value.status == T.TTQ_ERR_INVALID


# --------------------------------------------------------------- quantize

@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("bits,group", [(b, g) for b in (2, 3, 4, 5) for g in (16, 32, 64, 128)])
def test_quantize_parity(T, wdt, bits, group):
    say(f"quantize wdt={wdt} bits={bits} group={group}")
    M, K = 136, 1152
    rng = np.random.default_rng(bits * 1000 + group)
    W = synth.encode(rng.standard_normal((M, K)) * 0.02, wdt)
    s = (rng.lognormal(0, 0.7, K)).astype(np.float32)
    codes, sc, zz = T.ttq_quantize_groups(to_dev(W, wdt), f32_dev(s), bits, group)
    _check_rtn(codes, sc, zz, oracle.quant_values(W, wdt, s), bits, group)


@pytest.mark.parametrize("bits,group", [(4, 32), (3, 16)])
def test_quantize_large_weight(T, bits, group):
    # More than 2^25 bf16 weights: the quantizer takes 4-row batches; ragged
    # row count so that the last row block is partial.
    M, K = 2051, 16384
    say(f"quantize large M={M} K={K} bits={bits} group={group}")
    rng = np.random.default_rng(77 + bits)
    W = synth.encode(rng.standard_normal((M, K), dtype=np.float32) * 0.01, "bf16")
    s = (rng.lognormal(0, 0.5, K)).astype(np.float32)
    codes, sc, zz = T.ttq_quantize_groups(to_dev(W, "bf16"), f32_dev(s), bits, group)
    _check_rtn(codes, sc, zz, oracle.quant_values(W, "bf16", s), bits, group)


def test_quantize_without_scales_is_plain_rtn(T):
    say("quantize s=NULL")
    M, K = 64, 512
    rng = np.random.default_rng(9)
    W = synth.encode(rng.standard_normal((M, K)) * 0.05, "bf16")
    codes, sc, zz = T.ttq_quantize_groups(to_dev(W, "bf16"), None, 4, 32)
    v = oracle.quant_values(W, "bf16", np.ones(K, np.float32))
    _check_rtn(codes, sc, zz, v, 4, 32)
    # bf16 weights with s = 1 hit exact ties (v / step = k + 1/2) often: the
    # band admits either code there
    assert exact_ties(v, oracle.group_rtn(v, 4, 32)["delta"], 32).any()


def test_quantize_degenerate_groups(T):
    say("quantize zero / constant / one-sided groups")
    M, K = 8, 256
    W = np.zeros((M, K), np.float32)
    W[1] = 0.25                       # constant positive row
    W[2] = -0.5                       # constant negative row
    W[3, :32] = np.linspace(0, 1, 32)  # one-sided group
    W[4, 100] = 3.0                   # a lone spike
    codes, sc, zz = T.ttq_quantize_groups(to_dev(W, "f32"), f32_dev(np.ones(K)), 3, 32)
    _check_rtn(codes, sc, zz, oracle.quant_values(W, "f32", np.ones(K, np.float32)), 3, 32)


@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_quantize_nan_groups(T, wdt):
    # NaN weights: the group range ignores them and a NaN value gets code 0
    # (the oracle's rule); an all-NaN group takes the zero-range rule (step
    # 1, zero 0).  Mixed groups with NaN keep their other codes exact.
    say(f"quantize NaN groups {wdt}")
    M, K = 16, 512
    rng = np.random.default_rng(31)
    Wf = rng.standard_normal((M, K)) * 0.05
    Wf[0, :32] = np.nan                       # a whole group
    Wf[1, 5] = np.nan                         # one value of a group
    Wf[2, 64:128:3] = np.nan                  # scattered over two groups
    Wf[3, :] = np.nan                         # a whole row
    Wf[5, 200] = np.nan
    Wf[5, 201:224] = 0.0                      # NaN among zeros
    W = synth.encode(Wf, wdt)
    s = rng.lognormal(0, 0.3, K).astype(np.float32)
    for bits, group in ((4, 32), (3, 16), (2, 64)):
        v = oracle.quant_values(W, wdt, s)
        assert (oracle.group_rtn(v, bits, group)["q"][np.isnan(Wf)] == 0).all()
        codes, sc, zz = T.ttq_quantize_groups(to_dev(W, wdt), f32_dev(s), bits, group)
        _check_rtn(codes, sc, zz, v, bits, group)
        assert (oracle.unpack_codes(host(codes), bits, K)[np.isnan(Wf)] == 0).all()


@pytest.mark.parametrize("bits,group,rank", [(2, 32, 16), (3, 16, 8), (4, 64, 5), (5, 32, 32), (4, 32, 48),
                                            (2, 32, 64)])
def test_quantize_lowrank_parity(T, bits, group, rank):
    say(f"quantize lowrank bits={bits} group={group} rank={rank}")
    wl, d = _inputs("c5", T=32, K=1024, M=96)
    s = oracle.awq_scales(oracle.stats(d["X"], "bf16"), 32, 0.5, 1e-2)
    B, A = oracle.lowrank_factors(d["W"], "bf16", s, rank)
    codes, sc, zz = T.ttq_quantize_groups(to_dev(d["W"], "bf16"), f32_dev(s), bits, group,
                                          B=f32_dev(B), A=f32_dev(A))
    _check_rtn(codes, sc, zz, oracle.quant_values(d["W"], "bf16", s, B, A), bits, group)


# ------------------------------------------------------------------ qgemm

def _qgemm_case(T, key, Tn, K, M, bits, group, xdt, ydt, seed=0):
    wl, d = _inputs(key, seed=seed, T=Tn, K=K, M=M)
    X, W = d["X"], d["W"]
    s = oracle.awq_scales(oracle.stats(X, xdt), Tn, 0.5, 1e-2)
    r = oracle.group_rtn(oracle.quant_values(W, wl.wdtype, s), bits, group)
    w_hat = oracle.dequant(r["q"], r["delta"], r["zero"], group)
    ref = oracle.project(X, xdt, s, w_hat)
    codes = oracle.pack_codes(r["q"], bits)
    ws = T.workspace(Tn, K, M, bits, group)
    Y = T.ttq_qgemm(to_dev(X, xdt), f32_dev(s), i32_dev(codes), f16_dev(r["delta"]), f16_dev(r["zero"]),
                    M, bits, group, y_dtype=torch.float32 if ydt == "f32" else torch.bfloat16, ws=ws)
    got = host(Y)
    got = got.astype(np.float64) if ydt == "f32" else bf16_bits_to_f64(got)
    y_elementwise_check(got, X, xdt, s, r["q"], r["delta"], r["zero"], group,
                        valu=(Tn <= 4 and K % 128 == 0), y_bf16=(ydt == "bf16"))
    return got, ref


@pytest.mark.parametrize("bits,group,K", [(4, 32, 1056), (3, 16, 1056), (2, 64, 1088), (5, 128, 1152),
                                          (4, 16, 1024), (3, 128, 1024)])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_qgemm_parity(T, bits, group, K, xdt):
    key = "c1" if xdt == "f32" else "c2"
    say(f"qgemm bits={bits} group={group} K={K} xdt={xdt}")
    got, ref = _qgemm_case(T, key, 200, K, 300, bits, group, xdt, "f32")
    err = rel_fro(got, ref)
    assert err < (Y_TOL if xdt == "bf16" else 1e-4), err


@pytest.mark.parametrize("Tn,M", [(1, 128), (5, 302), (129, 130), (16, 64), (192, 130), (257, 302), (700, 77),
                                  (805, 8142)])   # the last one: 128 x 256 GEMM tiles with ragged T and M
def test_qgemm_ragged_and_bf16_output(T, Tn, M):
    say(f"qgemm ragged T={Tn} M={M}")
    for ydt, tol in (("f32", Y_TOL), ("bf16", Y_TOL_BF16_OUT)):
        got, ref = _qgemm_case(T, "c2", Tn, 512, M, 4, 32, "bf16", ydt, seed=Tn)
        assert rel_fro(got, ref) < tol


@pytest.mark.parametrize("K", [64, 128, 192, 320, 448])
def test_qgemm_short_k_wide_tiles(T, K):
    # 128 x 256 projection tiles (6144 rows x 1000 tokens: 192 tiles, the
    # last token tile ragged) with 1 to 7 K steps of 64: fewer steps than
    # the W~ ring has slots, and every remainder of the three-step unroll.
    say(f"qgemm short K={K}, 128x256 tiles")
    got, ref = _qgemm_case(T, "c2", 1000, K, 6144, 4, 32, "bf16", "f32", seed=K)
    assert rel_fro(got, ref) < Y_TOL


@pytest.mark.parametrize("Tn,M", [(300, 130), (600, 1024)])
def test_qgemm_split_k(T, Tn, M):
    # ttq_qgemm at prompt-sized T with few output tiles and K = 8192: the
    # projection runs as two K slices whose fp32 partials are added in order.
    say(f"qgemm split-K T={Tn} M={M}")
    for ydt, tol in (("f32", Y_TOL), ("bf16", Y_TOL_BF16_OUT)):
        got, ref = _qgemm_case(T, "c4", Tn, 8192, M, 4, 32, "bf16", ydt, seed=Tn)
        assert rel_fro(got, ref) < tol


@pytest.mark.parametrize("Tn", [1, 3, 5, 8, 12, 16, 17, 33, 64, 65, 128])
@pytest.mark.parametrize("bits,group", [(4, 32), (3, 16), (2, 64), (5, 128)])
def test_qgemv_parity(T, Tn, bits, group):
    # The few-token kernel (T <= 128, K % 128 == 0): K = 1152 gives the 16
    # waves of a workgroup unequal chunk counts, M = 200 a partial row tile.
    say(f"qgemv T={Tn} bits={bits} group={group}")
    for xdt in ("bf16", "f32"):
        key = "c1" if xdt == "f32" else "c2"
        got, ref = _qgemm_case(T, key, Tn, 1152, 200, bits, group, xdt, "f32", seed=Tn + bits)
        err = rel_fro(got, ref)
        assert err < (Y_TOL if xdt == "bf16" else 1e-4), (xdt, err)


@pytest.mark.parametrize("Tn", [5, 7, 16])
@pytest.mark.parametrize("group,K,M", [(32, 1152, 200), (64, 1152, 203), (128, 2048, 77), (32, 18432, 33),
                                       (64, 256, 8200), (32, 14336, 1000)])
def test_qgemv_group_sums(T, Tn, group, K, M):
    # 4-bit codes, 5 <= T <= 16, bf16 X: the group scale applied to sums on
    # the matrix cores (x * (1/s) rounded once to bf16 in LDS, codes exact as
    # 128 + code); fp32 X takes the per-weight expansion.  K = 1152: nine
    # chunks, the last 512-channel set partial, three K slices; M = 203 / 77
    # / 33 partial 64-row blocks; K = 18432, M = 33: 36 slices; K = 256,
    # M = 8200: one slice (no partials), half a set; K = 14336, M = 1000: two
    # sets (two waves) per slice, 14 slices.
    say(f"qgemv group sums T={Tn} group={group} K={K} M={M}")
    for xdt in ("bf16", "f32"):
        key = "c1" if xdt == "f32" else "c2"
        for ydt in ("f32", "bf16"):
            got, ref = _qgemm_case(T, key, Tn, K, M, 4, group, xdt, ydt, seed=Tn + group)
            tol = Y_TOL if ydt == "f32" else Y_TOL_BF16_OUT
            assert rel_fro(got, ref) < tol, (xdt, ydt)


@pytest.mark.parametrize("Tn", [1, 2, 3, 4])
@pytest.mark.parametrize("bits,group,K", [(4, 32, 1152), (4, 32, 4224), (3, 16, 4224), (2, 64, 18432),
                                          (5, 128, 4224), (4, 16, 2048), (2, 128, 1152),
                                          (4, 32, 14336), (3, 64, 8320)])
def test_qgemv_few_tokens(T, Tn, bits, group, K):
    # One to four tokens run on the vector ALUs in fp32 (no bf16 rounding of
    # weights or tokens), so the bar is fp32 accumulation, not 2e-3.  K = 1152
    # and 4224 end in a partial 2048-channel piece; K = 18432 gives 9 pieces
    # over 5 waves; M = 203 a partial 8-row block.
    say(f"qgemv few tokens T={Tn} bits={bits} group={group} K={K}")
    for xdt in ("bf16", "f32"):
        key = "c1" if xdt == "f32" else "c2"
        got, ref = _qgemm_case(T, key, Tn, K, 203, bits, group, xdt, "f32", seed=Tn + 7 * bits)
        err = rel_fro(got, ref)
        assert err < 2e-5, (xdt, err)


@pytest.mark.parametrize("Tn", [1, 2, 3, 4])
@pytest.mark.parametrize("bits,group,xdt", [(4, 32, "bf16"), (3, 16, "bf16"), (2, 64, "f32")])
def test_qgemm_batched_prompts(T, Tn, bits, group, xdt):
    # One launch for several prompts, each with its own quantized state: every
    # prompt's Y matches the oracle and, bit for bit, its own ttq_qgemm call.
    say(f"qgemm batched P=5 T={Tn} bits={bits} group={group} {xdt}")
    P, K, M = 5, 1152, 203
    key = "c1" if xdt == "f32" else "c2"
    Xs, ss, cs, ds, zs, refs = [], [], [], [], [], []
    for pi in range(P):
        wl, d = _inputs(key, seed=100 + pi, T=Tn, K=K, M=M)
        sp = oracle.awq_scales(oracle.stats(d["X"], xdt), Tn, 0.5, 1e-2)
        r = oracle.group_rtn(oracle.quant_values(d["W"], wl.wdtype, sp), bits, group)
        refs.append(oracle.project(d["X"], xdt, sp, oracle.dequant(r["q"], r["delta"], r["zero"], group)))
        Xs.append(to_dev(d["X"], xdt)); ss.append(f32_dev(sp)); cs.append(i32_dev(oracle.pack_codes(r["q"], bits)))
        ds.append(f16_dev(r["delta"])); zs.append(f16_dev(r["zero"]))
    Y = T.ttq_qgemm_batched(torch.stack(Xs), torch.stack(ss), torch.stack(cs), torch.stack(ds), torch.stack(zs),
                            M, bits, group)
    Yh = host(Y)
    for pi in range(P):
        assert rel_fro(Yh[pi], refs[pi]) < 2e-5
        one = T.ttq_qgemm(Xs[pi], ss[pi], cs[pi], ds[pi], zs[pi], M, bits, group)
        np.testing.assert_array_equal(host(one), Yh[pi])


def test_largest_K(T):
    # K = 2^18, the largest K the library accepts (4096 channel blocks of 64
    # for the shrinkage mean): statistics, fused scales, quantization and the
    # projection for one, two and eight tokens.
    say("largest K = 2^18")
    # The state is checked against the oracle (codes band-aware), Y element-
    # wise against the projection of the library's own state (the fp32 bound
    # for T <= 2) and against the oracle at the 2e-3 bar: with 4M codes, an
    # in-band code difference moves a few outputs by ~1e-4 relative.
    K, M = 1 << 18, 16
    for Tn in (1, 2, 8):
        wl, d = _inputs("c2", seed=50 + Tn, T=Tn, K=K, M=M)
        ref = oracle.linear(d["X"], "bf16", d["W"], "bf16", 4, 32, 0.5, 1e-2)
        Y, st = _run_linear(T, wl, d)
        _check_linear_state(wl, d, st, ref)
        _check_y_on_state(wl, d, Y, st)
        assert rel_fro(host(Y), ref["Y"]) < Y_TOL


@pytest.mark.parametrize("Tn", [8, 12, 16])
def test_qgemm_few_tokens_beyond_16384_channels(T, Tn):
    # K above the matrix-core few-token kernel's limit: T = 8 falls back to
    # the tile kernel, T = 12 and 16 take the split-K path.
    say(f"qgemm T={Tn} K=18432")
    got, ref = _qgemm_case(T, "c2", Tn, 18432, 96, 4, 32, "bf16", "f32", seed=Tn)
    assert rel_fro(got, ref) < Y_TOL


def test_qgemm_identity_input_layout(T):
    # X = I: Y[t][o] = bf16((q - z) * step / s_t), element by element.
    say("qgemm identity layout")
    K, M = 256, 96
    rng = np.random.default_rng(3)
    W = synth.encode(rng.standard_normal((M, K)) * 0.05, "bf16")
    s = rng.lognormal(0, 0.5, K).astype(np.float32)
    r = oracle.group_rtn(oracle.quant_values(W, "bf16", s), 4, 32)
    w_eff = oracle.dequant(r["q"], r["delta"], r["zero"], 32) / s.astype(np.float64)[None, :]
    X = synth.encode(np.eye(K), "bf16")
    ws = T.workspace(K, K, M, 4, 32)
    Y = T.ttq_qgemm(to_dev(X, "bf16"), f32_dev(s), i32_dev(oracle.pack_codes(r["q"], 4)),
                    f16_dev(r["delta"]), f16_dev(r["zero"]), M, 4, 32, ws=ws)
    got = host(Y).astype(np.float64)
    np.testing.assert_allclose(got, w_eff.T, rtol=2.0 ** -8, atol=1e-30)


# ---------------------------------------------------------------- lowrank

def _offset_dev(a: np.ndarray) -> torch.Tensor:
    """fp32 device copy whose data starts 4 bytes past a 16-byte boundary."""
    buf = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).ravel()).to("cuda")
    return buf[1:].view(a.shape)


@pytest.mark.parametrize("xdt,rank,a_off,K", [("bf16", 16, False, 512), ("f32", 7, False, 512),
                                              ("bf16", 32, False, 512), ("bf16", 16, True, 512),
                                              ("bf16", 5, False, 512), ("bf16", 16, False, 4096),
                                              ("bf16", 64, False, 512), ("f32", 40, False, 512)])
def test_lowrank_add_parity(T, xdt, rank, a_off, K):
    # bf16 X with an aligned A runs Z on the matrix cores; fp32 X or an A
    # that is not 16-byte aligned runs the K-slice kernel.  K = 4096 with 150
    # tokens (10 token tiles) splits the matrix-core Z into 8 K slices.
    say(f"lowrank_add xdt={xdt} rank={rank} A offset={a_off} K={K}")
    rng = np.random.default_rng(rank)
    Tn, M = 150, 200
    X = synth.encode(rng.standard_normal((Tn, K)), xdt)
    A = (rng.standard_normal((rank, K)) * 0.05).astype(np.float32)
    B = (rng.standard_normal((M, rank))).astype(np.float32)
    Y0 = rng.standard_normal((Tn, M)).astype(np.float32)
    x = oracle.decode(X, xdt)
    ref = Y0.astype(np.float64) + (x @ A.astype(np.float64).T) @ B.astype(np.float64).T
    Y = f32_dev(Y0)
    ws = T.workspace(Tn, K, M, 2, 32, rank)
    T.ttq_lowrank_add(to_dev(X, xdt), _offset_dev(A) if a_off else f32_dev(A), f32_dev(B), Y, ws=ws)
    got = host(Y)
    assert rel_fro(got, ref) < 1e-5
    assert rel_fro(got.astype(np.float64) - Y0, ref - Y0) < 1e-5     # the low-rank term itself


# ------------------------------------------------------------ end to end

E2E = [
    ("c1", dict()),
    ("c2", dict(T=160, K=1024, M=288)),
    ("c3", dict(T=96, K=1024, M=320)),
    ("c4", dict(T=100, K=2048, M=256)),
    ("c5", dict(T=128, K=512, M=512)),
    # prompt-sized T: the quantizer writes the dequantized weight, matrix-core GEMM
    ("c2-long", dict(T=300, K=1024, M=288)),
    ("c3-long", dict(T=400, K=1024, M=320)),
    ("c4-long", dict(T=256, K=2048, M=256)),
    ("c5-long", dict(T=260, K=512, M=512)),
    # low-rank Z split into 4 K slices, summed in the GEMM epilogue
    ("c5-slices", dict(T=300, K=2048, M=256)),
    # few 128 x 256 tiles and K >= 8192: two K slices plus their ordered sum
    ("c4-split", dict(T=260, K=8192, M=302)),
    # ranks above 32: the GEMM epilogue adds Z B^T in two chunks of ranks
    ("c5-rank64", dict(T=260, K=512, M=512, rank=64)),
    ("c5-rank40", dict(T=64, K=512, M=320, rank=40)),
]


def _check_linear_state(wl, d, st, ref, B=None, A=None):
    """The prompt state left by ttq_linear: statistics and scales against the
    oracle, then (whatever the scales) the quantizer's codes, steps and zeros
    against the oracle's group RTN on the library's own scales."""
    np.testing.assert_allclose(host(st["ssq"]), ref["ssq"], rtol=1e-12)
    s = host(st["s"])
    check_scales(s, ref["s"], rtol=S_TOL)
    check_quant_state(host(st["codes"]), host(st["scale_f16"]), host(st["zero_f16"]), d["W"], wl.wdtype, s,
                      wl.bits, wl.group, B, A)


def _check_y_on_state(wl, d, Y, st, B=None, A=None):
    """Every element of Y against the projection of the library's own state."""
    q = oracle.unpack_codes(host(st["codes"]), wl.bits, wl.K)
    y_elementwise_check(host(Y), d["X"], wl.xdtype, host(st["s"]), q, host(st["scale_f16"]).view(np.float16),
                        host(st["zero_f16"]).view(np.float16), wl.group, B, A,
                        valu=(wl.T <= 4 and wl.K % 128 == 0))


def _run_linear(T, wl, d, B=None, A=None):
    dev_x = to_dev(d["X"], wl.xdtype)
    dev_w = to_dev(d["W"], wl.wdtype)
    st = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
    Y = T.ttq_linear(dev_x, dev_w, wl.bits, wl.group, wl.alpha, wl.lambda_rel,
                     B=None if B is None else f32_dev(B), A=None if A is None else f32_dev(A), state=st)
    return Y, st


@pytest.mark.parametrize("key,sizes", E2E, ids=[k for k, _ in E2E])
def test_linear_end_to_end(T, key, sizes):
    say(f"linear e2e {key} {sizes}")
    wl, d = _inputs(key.split("-")[0], **sizes)
    B = A = None
    if wl.rank:
        s0 = oracle.awq_scales(oracle.stats(d["X"], wl.xdtype), wl.T, wl.alpha, wl.lambda_rel)
        B, A = oracle.lowrank_factors(d["W"], wl.wdtype, s0, wl.rank)
    ref = oracle.linear(d["X"], wl.xdtype, d["W"], wl.wdtype, wl.bits, wl.group, wl.alpha,
                        wl.lambda_rel, B=B, A=A)
    Y, st = _run_linear(T, wl, d, B, A)
    _check_linear_state(wl, d, st, ref, B, A)
    err = rel_fro(host(Y), ref["Y"])
    say(f"  Y rel err {err:.3e}")
    assert err < Y_TOL
    _check_y_on_state(wl, d, Y, st, B, A)


@pytest.mark.parametrize("p,key,sizes", [(1.0, "c2", dict(T=400, K=1024, M=300)),
                                          (3.0, "c1", dict(T=64, K=768, M=200)),
                                          (0.5, "c3", dict(T=256, K=2048, M=160))])
def test_linear_moment_p(T, p, key, sizes):
    # The whole layer with a moment order other than 2: statistics, the
    # lambda and scales fused into the quantizer, codes and Y.
    say(f"linear p={p} {key} {sizes}")
    wl, d = _inputs(key, **sizes)
    ref = oracle.linear(d["X"], wl.xdtype, d["W"], wl.wdtype, wl.bits, wl.group, wl.alpha,
                        wl.lambda_rel, p=p)
    st = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
    Y = T.ttq_linear(to_dev(d["X"], wl.xdtype), to_dev(d["W"], wl.wdtype), wl.bits, wl.group, wl.alpha,
                     wl.lambda_rel, p=p, state=st)
    _check_linear_state(wl, d, st, ref)
    s = host(st["s"])
    assert rel_fro(host(Y), ref["Y"]) < (Y_TOL if wl.xdtype == "bf16" else 1e-4)
    _check_y_on_state(wl, d, Y, st)
    # the fused scales equal the standalone call's bit for bit
    s2 = T.ttq_awq_scales(st["ssq"], wl.T, wl.alpha, wl.lambda_rel, p=p)
    np.testing.assert_array_equal(host(s2), s)


@pytest.mark.parametrize("key,sizes", [("c2", dict(T=300, K=1024)), ("c1", dict(T=96, K=768))])
def test_linear_shared_statistics(T, key, sizes):
    # q/k/v-like layers on one X: one statistics pass, then each layer; every
    # output and state equals its own ttq_linear call bit for bit, and Y
    # matches the oracle.
    say(f"linear shared {key} {sizes}")
    wl, d = _inputs(key, M=256, **sizes)
    rng = np.random.default_rng(77)
    shapes = [(256, 4, 32), (128, 3, 16), (192, 2, 64)]
    X = to_dev(d["X"], wl.xdtype)
    Ws = [synth.encode(rng.standard_normal((m, wl.K)) * 0.02, wl.wdtype) for m, _, _ in shapes]
    layers, refs = [], []
    for (m, b, g), Wh in zip(shapes, Ws):
        st = T.linear_state(wl.T, wl.K, m, b, g)
        if layers:
            st["ssq"] = None
        layers.append(dict(W=to_dev(Wh, wl.wdtype), bits=b, group=g, state=st))
        refs.append(oracle.linear(d["X"], wl.xdtype, Wh, wl.wdtype, b, g, wl.alpha, wl.lambda_rel))
    Ys = T.ttq_linear_shared(X, layers, wl.alpha, wl.lambda_rel)
    tol = Y_TOL if wl.xdtype == "bf16" else 1e-4
    for (m, b, g), ly, Y, ref in zip(shapes, layers, Ys, refs):
        assert rel_fro(host(Y), ref["Y"]) < tol
        st1 = T.linear_state(wl.T, wl.K, m, b, g)
        Y1 = T.ttq_linear(X, ly["W"], b, g, wl.alpha, wl.lambda_rel, state=st1)
        np.testing.assert_array_equal(host(Y1), host(Y))
        for k in ("s", "codes", "scale_f16", "zero_f16"):
            np.testing.assert_array_equal(host(st1[k]), host(ly["state"][k]))
    np.testing.assert_allclose(host(layers[0]["state"]["ssq"]), refs[0]["ssq"], rtol=1e-12)


def test_linear_lowrank_unaligned_factor(T):
    # Prompt-sized T with an A that is not 16-byte aligned: the low-rank term
    # is added by the standalone kernels after the GEMM instead of its epilogue.
    say("linear low-rank, unaligned A")
    wl, d = _inputs("c5", T=260, K=512, M=512)
    s0 = oracle.awq_scales(oracle.stats(d["X"], wl.xdtype), wl.T, wl.alpha, wl.lambda_rel)
    B, A = oracle.lowrank_factors(d["W"], wl.wdtype, s0, wl.rank)
    ref = oracle.linear(d["X"], wl.xdtype, d["W"], wl.wdtype, wl.bits, wl.group, wl.alpha,
                        wl.lambda_rel, B=B, A=A)
    Y = T.ttq_linear(to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16"), wl.bits, wl.group, wl.alpha,
                     wl.lambda_rel, B=f32_dev(B), A=_offset_dev(A))
    assert rel_fro(host(Y), ref["Y"]) < Y_TOL
    Y2, _ = _run_linear(T, wl, d, B, A)     # aligned: fused epilogue
    assert rel_fro(host(Y2), host(Y)) < 1e-5


def test_linear_lowrank_streamed_stage(T):
    # A residual layer whose staged w~ exceeds 64 MiB (8192 x 4608 bf16,
    # 75.5 MB): the residual quantizer writes w~ by streaming stores.  Its
    # codes, steps and zeros must equal the standalone quantizer's (which
    # stages nothing) bit for bit; Y must equal the projection of that state
    # plus the low-rank term, and the oracle on sampled rows.
    say("linear low-rank, streamed w~ (8192 x 4608, rank 8)")
    wl, d = _inputs("c5", T=256, K=4608, M=8192)
    rng = np.random.default_rng(7)
    B = (rng.standard_normal((wl.M, 8)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((8, wl.K)) * 0.02).astype(np.float32)
    Y, st = _run_linear(T, wl, d, B, A)
    dev_w = to_dev(d["W"], wl.wdtype)
    codes, scale, zero = T.ttq_quantize_groups(dev_w, st["s"], wl.bits, wl.group, B=f32_dev(B), A=f32_dev(A))
    assert torch.equal(codes, st["codes"])
    assert torch.equal(scale.view(torch.int16), st["scale_f16"].view(torch.int16))
    assert torch.equal(zero.view(torch.int16), st["zero_f16"].view(torch.int16))
    dev_x = to_dev(d["X"], wl.xdtype)
    ws = T.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group, rank=8)
    Yq = T.ttq_qgemm(dev_x, st["s"], st["codes"], st["scale_f16"], st["zero_f16"], wl.M, wl.bits, wl.group, ws=ws)
    T.ttq_lowrank_add(dev_x, f32_dev(A), f32_dev(B), Yq, ws=ws)
    assert rel_fro(host(Yq), host(Y)) < 1e-5
    rows = np.array([0, 1, 2047, 4096, 6000, wl.M - 1])
    ref = oracle.linear(d["X"], wl.xdtype, d["W"], wl.wdtype, wl.bits, wl.group, wl.alpha, wl.lambda_rel,
                        B=B, A=A, rows=rows)
    err = rel_fro(host(Y)[:, rows], ref["Y"])
    say(f"  Y rel err (sampled rows) {err:.3e}")
    assert err < Y_TOL


def test_decode_steps_reuse_prompt_state(T):
    say("decode steps")
    wl, d = _inputs("c4", T=64, K=2048, M=256, decode_T=(1, 4, 16))
    ref = oracle.linear(d["X"], "bf16", d["W"], "bf16", wl.bits, wl.group, wl.alpha, wl.lambda_rel)
    _, st = _run_linear(T, wl, d)
    ws = T.workspace(16, wl.K, wl.M, wl.bits, wl.group)
    for td, Xd in d["X_decode"].items():
        Yd = T.ttq_qgemm(to_dev(Xd, "bf16"), st["s"], st["codes"], st["scale_f16"], st["zero_f16"],
                         wl.M, wl.bits, wl.group, ws=ws)
        refd = oracle.project(Xd, "bf16", ref["s"], ref["w_hat"])
        assert rel_fro(host(Yd), refd) < Y_TOL, td


@pytest.mark.parametrize("key,sizes", [("c3", dict(T=384, K=1024, M=320)), ("c4", dict(T=300, K=8192, M=260))])
def test_linear_and_qgemm_share_the_dequantized_weight(T, key, sizes):
    # For prompt-sized T the whole-layer call takes the dequantized weight
    # from the quantizer, ttq_qgemm expands the stored codes itself; both
    # must produce the same bf16 weight, hence bitwise the same Y (the
    # second shape runs the projection as two K slices).
    say(f"linear vs qgemm on the prompt state {key} {sizes}")
    wl, d = _inputs(key, **sizes)
    Y, st = _run_linear(T, wl, d)
    ws = T.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group)
    Yq = T.ttq_qgemm(to_dev(d["X"], "bf16"), st["s"], st["codes"], st["scale_f16"], st["zero_f16"],
                     wl.M, wl.bits, wl.group, ws=ws)
    assert torch.equal(Y, Yq)


def test_linear_stage_events(T):
    # Events recorded inside ttq_linear do not change the result and time
    # every stage of the call.
    say("linear stage events")
    wl, d = _inputs("c2", T=512, K=1024, M=512)
    Y0, _ = _run_linear(T, wl, d)
    ev = T.StageEvents()
    st = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
    Y1 = T.ttq_linear(to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16"), wl.bits, wl.group, wl.alpha,
                      wl.lambda_rel, state=st, stage_events=ev)
    ms = ev.stage_ms()
    assert set(ms) == set(T.LINEAR_STAGES)
    assert all(v >= 0.0 for v in ms.values()) and ms["projection"] > 0.0
    assert torch.equal(Y0, Y1)


def test_linear_graph_replay(T):
    # The whole-layer call captured in a graph (no memset nodes: the reduction
    # counter is reset by the statistics kernel itself) and replayed several
    # times with unrelated eager work in between; every replay must equal the
    # eager result bitwise.
    say("linear graph replay")
    wl, d = _inputs("c2", T=300, K=1024, M=288)
    X, W = to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16")
    st = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
    ws = T.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group)
    Y = torch.empty((wl.T, wl.M), dtype=torch.float32, device="cuda")
    T.ttq_linear(X, W, wl.bits, wl.group, wl.alpha, wl.lambda_rel, Y=Y, ws=ws, state=st)
    torch.cuda.synchronize()
    ref = Y.clone()
    ref_state = {k: v.clone() for k, v in st.items()}
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cs):
        T.ttq_linear(X, W, wl.bits, wl.group, wl.alpha, wl.lambda_rel, Y=Y, ws=ws, state=st)
    torch.cuda.synchronize()
    for rep in range(4):
        Y.fill_(float("nan"))
        for v in st.values():
            v.zero_()
        ws.fill_(0xA5)                      # stale scratch, including the counter
        junk = torch.randn(1000, device="cuda") * 2
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), rep
        for k in st:
            assert torch.equal(st[k], ref_state[k]), (rep, k)
        assert torch.isfinite(junk).all()


def test_run_twice_bitwise_identical(T):
    say("determinism")
    wl, d = _inputs("c3", T=96, K=1024, M=320)
    Y1, st1 = _run_linear(T, wl, d)
    Y2, st2 = _run_linear(T, wl, d)
    assert torch.equal(Y1, Y2)
    for k in st1:
        assert torch.equal(st1[k], st2[k]), k


@pytest.mark.parametrize("Tn", [70, 300])
def test_linear_strided_operands(T, Tn):
    say(f"linear strided X/W/Y T={Tn}")
    wl, d = _inputs("c2", T=Tn, K=512, M=200)
    X = torch.zeros((Tn, 512 + 64), dtype=torch.bfloat16, device="cuda")
    X[:, :512] = to_dev(d["X"], "bf16")
    W = torch.zeros((200, 512 + 32), dtype=torch.bfloat16, device="cuda")
    W[:, :512] = to_dev(d["W"], "bf16")
    Yb = torch.full((Tn, 200 + 28), 5.0, dtype=torch.float32, device="cuda")
    T.ttq_linear(X[:, :512], W[:, :512], wl.bits, wl.group, wl.alpha, wl.lambda_rel, Y=Yb[:, :200])
    ref = oracle.linear(d["X"], "bf16", d["W"], "bf16", wl.bits, wl.group, wl.alpha, wl.lambda_rel)
    got = host(Yb)
    assert rel_fro(got[:, :200], ref["Y"]) < Y_TOL
    assert np.all(got[:, 200:] == 5.0)   # padding columns untouched


def test_empty_calls_are_noops(T):
    say("empty calls")
    Y = torch.full((0, 64), 1.0, device="cuda")
    X = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    T.ttq_linear(X, W, 4, 32, 0.5, 1e-2, Y=Y, ws=torch.empty(256, dtype=torch.uint8, device="cuda"))
    ssq = torch.full((256,), 3.0, dtype=torch.float64, device="cuda")
    T.ttq_stats(X, ssq, accumulate=True)
    assert torch.all(ssq == 3.0)
    T.ttq_stats(X, ssq, accumulate=False)
    assert torch.all(ssq == 0.0)


def test_binding_raises_on_bad_arguments(T):
    X = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((8, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises((T.TTQError, ValueError)):
        T.ttq_linear(X, W, 4, 32, 0.5, 1e-2)
    with pytest.raises(TypeError):
        T.ttq_stats(torch.zeros((4, 64)), torch.zeros(64, dtype=torch.float64))


def test_side_stream_temporaries(T):
    # Calls on a stream other than the current one: the binding's default
    # workspace and outputs are allocated on the launch stream, so work queued
    # meanwhile on the current stream cannot reuse that memory while the
    # kernels still run.  The results equal the current-stream call's.
    say("side-stream launch")
    wl, d = _inputs("c2", T=300, K=1024, M=288)
    X, W = to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16")
    Y0 = T.ttq_linear(X, W, wl.bits, wl.group, wl.alpha, wl.lambda_rel)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for handle in (side, side.cuda_stream):
        Y1 = T.ttq_linear(X, W, wl.bits, wl.group, wl.alpha, wl.lambda_rel, stream=handle)
        # the current stream allocates and overwrites memory while side runs
        junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
        del junk
        codes, sc, zz = T.ttq_quantize_groups(W, None, 4, 32, stream=handle)
        outs.append((Y1, codes))
    side.synchronize()
    torch.cuda.synchronize()
    ref_codes = T.ttq_quantize_groups(W, None, 4, 32)[0]
    for Y1, codes in outs:
        assert torch.equal(Y1, Y0)
        assert torch.equal(codes, ref_codes)
