"""ttq_linear_noalloc: the whole-layer call with the library's own scratch
array as its workspace, through the C ABI (raw ctypes).

Two calls in a row on one GPU, the second with a smaller layer, each checked
against ttq_linear on the same inputs (bitwise: the same kernels on the same
bytes) and against the oracle (scales, quantizer state, Y within the bars of
tests/test_gpu_parity.py).  A layer whose workspace exceeds the array is
rejected before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_quant_state, check_scales, host, rel_fro, say, to_dev
from online_activation_aware_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    from online_activation_aware_amd import ttq
    ttq.lib()
    return ttq


def _args(T, X, W, wl, Y, st):
    return T.LinearArgs(
        X=X.data_ptr(), xt=T.TTQ_BF16 if X.dtype == torch.bfloat16 else T.TTQ_F32, T=X.shape[0], K=X.shape[1],
        ldx=X.stride(0), W=W.data_ptr(), wt=T.TTQ_BF16 if W.dtype == torch.bfloat16 else T.TTQ_F32,
        M=W.shape[0], ldw=W.stride(0), alpha=wl.alpha, lambda_rel=wl.lambda_rel, p=2.0, bits=wl.bits,
        group=wl.group, B=None, A=None, rank=0, Y=Y.data_ptr(), yt=T.TTQ_F32, ldy=Y.stride(0),
        ssq=st["ssq"].data_ptr(), s=st["s"].data_ptr(), codes=st["codes"].data_ptr(),
        scale_f16=st["scale_f16"].data_ptr(), zero_f16=st["zero_f16"].data_ptr(), stage_events=None)


def test_noalloc_matches_linear_twice(T):
    L = T.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # the first layer takes the prompt-sized projection (dequantized weight in
    # the scratch array), the second, smaller one the few-token kernels
    for key, sizes in (("c2", dict(T=300, K=1024, M=288)), ("c3", dict(T=96, K=512, M=160))):
        wl = synth.workload(key, **sizes)
        say(f"noalloc {key} {sizes}")
        d = synth.make_inputs(wl)
        X, W = to_dev(d["X"], wl.xdtype), to_dev(d["W"], wl.wdtype)
        st_ref = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
        Y_ref = T.ttq_linear(X, W, wl.bits, wl.group, wl.alpha, wl.lambda_rel, state=st_ref)
        st = T.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group)
        Y = torch.full((wl.T, wl.M), float("nan"), dtype=torch.float32, device="cuda")
        a = _args(T, X, W, wl, Y, st)
        assert L.ttq_linear_noalloc(ctypes.byref(a), stream) == T.TTQ_OK, L.ttq_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref)
        for k in st:
            assert torch.equal(st[k], st_ref[k]), k
        ref = oracle.linear(d["X"], wl.xdtype, d["W"], wl.wdtype, wl.bits, wl.group, wl.alpha, wl.lambda_rel)
        np.testing.assert_allclose(host(st["ssq"]), ref["ssq"], rtol=1e-12)
        s = host(st["s"])
        check_scales(s, ref["s"])
        check_quant_state(host(st["codes"]), host(st["scale_f16"]), host(st["zero_f16"]), d["W"], wl.wdtype, s,
                          wl.bits, wl.group)
        assert rel_fro(host(Y), ref["Y"]) < 2e-3


def test_noalloc_rejects_layers_beyond_the_array(T):
    L = T.lib()
    cap = 64 << 20
    # 8192 x 8192 at T = 2048 needs the 128 MiB dequantized weight
    assert T.ttq_workspace_bytes(2048, 8192, 8192, 4, 32, 0) > cap
    fake = 0x100000   # aligned, never dereferenced: the check fails first
    a = T.LinearArgs(X=fake, xt=T.TTQ_BF16, T=2048, K=8192, ldx=8192, W=fake, wt=T.TTQ_BF16, M=8192, ldw=8192,
                     alpha=0.5, lambda_rel=0.01, p=2.0, bits=4, group=32, B=None, A=None, rank=0, Y=fake,
                     yt=T.TTQ_F32, ldy=8192, ssq=None, s=None, codes=None, scale_f16=None, zero_f16=None,
                     stage_events=None)
    assert L.ttq_linear_noalloc(ctypes.byref(a), None) == T.TTQ_ERR_INVALID
    assert b"TTQ_NOALLOC_SCRATCH_BYTES" in L.ttq_last_error()
