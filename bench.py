#!/usr/bin/env python3
"""Benchmark of the TTQ per-prompt layer path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|c1..c5]

A step is one pass of the whole per-prompt path for one linear layer —
activation statistics -> shrunk AWQ scales -> group RTN of the scaled weight
-> quantized projection (plus the low-rank term when the workload has one) —
through the C ABI's ttq_linear, on synthetic inputs already resident in HBM.
Inputs rotate over several copies (>= 1 GiB in total) so that successive
steps do not find X and W in the 256 MiB Infinity Cache.

By default the 4096->4096, T = 2048 layer is the headline (the JSON line's
value, roofline and CPU baseline), and the other four workloads (768->768
fp32; 4096->14336; 14336->4096 with its decode steps and batched decode;
the low-rank 4096->4096 layer with its per-prompt factors) are timed in the
same run under "workloads".

Prints one JSON line (stdout): the layer time in microseconds, the roofline
of the dominant kernel (the projection GEMM) from HIP events that ttq_linear
records on its stream in every timed step, the per-stage breakdown, and the
CPU oracle timed on the host.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ttq_linear µs/layer (stats+quant+qGEMM); qGEMM TFLOP/s; HBM GB/s vs peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)

# HBM bytes per projection-GEMM launch measured with rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE, scaled by the factor a plain copy of known size gives), keyed by
# the SHA-256 of the kernel source they were taken on.  A source change
# invalidates them (traffic is then reported as null).
MEASURED_TRAFFIC = {
    # 4096->4096, T=2048 layer: profiles/ttq_linear_4096x4096_t2048_b4g32_pmc_traffic.txt
    "6c1ab95eb15a86b8": {"workload": "c2", "fetch_bytes": 134378945, "write_bytes": 35414221,
                         "fetch_factor": 1.9999, "write_factor": 1.0},
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the GEMM source's code (comments and blank lines dropped), so
    that the stored traffic counters go stale when the kernel changes."""
    import re
    path = os.path.join(ROOT, "online_activation_aware_amd", "csrc", "gemm_bf16.hip")
    with open(path, encoding="utf-8") as f:
        text = f.read()
    code = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
    return hashlib.sha256("\n".join(l for l in code if l).encode()).hexdigest()[:16]


def esize(dt: str) -> int:
    return 4 if dt == "f32" else 2


def algorithmic_bytes(wl) -> dict:
    """Bytes each stage must move at minimum (Y in fp32): statistics read X
    and write ssq; the quantizer reads W (and the factors) and ssq, writes s,
    codes, steps and zeros; the projection reads X, codes, steps, zeros and s
    and writes Y."""
    T, K, M, b, g = wl.T, wl.K, wl.M, wl.bits, wl.group
    codes = M * K * b // 8
    steps = 2 * M * (K // g) * 2
    return {
        "stats": T * K * esize(wl.xdtype) + K * 8,
        "quantize": M * K * esize(wl.wdtype) + K * 8 + K * 4 + codes + steps
        + (wl.rank * (M + K) * 4 if wl.rank else 0),
        "projection": T * K * esize(wl.xdtype) + K * 4 + codes + steps + T * M * 4,
    }


def time_factors(ttq, Ws, s, om, wl, l, q, args) -> dict:
    """ttq_lowrank_factors over the rotating weight copies, one call per copy
    captured in a HIP graph (its small kernels are launch-bound eagerly)."""
    import torch
    n = len(Ws)
    Bf = torch.empty((wl.M, wl.rank), dtype=torch.float32, device=s.device)
    Af = torch.empty((wl.rank, wl.K), dtype=torch.float32, device=s.device)
    wsf = torch.empty(ttq.lib().ttq_lowrank_factors_workspace_bytes(wl.M, wl.K, l), dtype=torch.uint8,
                      device=s.device)

    def calls():
        for W in Ws:
            ttq.ttq_lowrank_factors(W, s, om, wl.rank, q, B=Bf, A=Af, ws=wsf)
    calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        calls()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(args.steps / n))
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (reps * n) * 1e3
    passes = 2 * q + 2
    wbytes = wl.M * wl.K * 2
    return {"us": round(us, 2), "l": l, "q": q, "passes_over_w": passes,
            "method": "randomized subspace iteration (CholQR2, Jacobi), bf16 transpose of W once",
            "w_stream_gbs": round((passes + 2) * wbytes / (us * 1e-6) / 1e9, 1)}


def cpu_baseline(wl, data, B=None, A=None) -> dict:
    """The CPU oracle, as it stands, timed on this host on the same layer."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    times, stages = [], {"stats_scales": [], "quantize": [], "projection": []}
    t_start = time.perf_counter()
    while len(times) < 64 and (len(times) < 3 or time.perf_counter() - t_start < 10.0):
        t0 = time.perf_counter()
        ssq = oracle.stats(data["X"], wl.xdtype)
        s = oracle.awq_scales(ssq, wl.T, wl.alpha, wl.lambda_rel)
        t1 = time.perf_counter()
        v = oracle.quant_values(data["W"], wl.wdtype, s, B, A)
        r = oracle.group_rtn(v, wl.bits, wl.group)
        oracle.pack_codes(r["q"], wl.bits)
        t2 = time.perf_counter()
        w_hat = oracle.dequant(r["q"], r["delta"], r["zero"], wl.group)
        Y = oracle.project(data["X"], wl.xdtype, s, w_hat, B, A)
        t3 = time.perf_counter()
        times.append(t3 - t0)
        stages["stats_scales"].append(t1 - t0)
        stages["quantize"].append(t2 - t1)
        stages["projection"].append(t3 - t2)
        assert np.isfinite(Y).all()
    dt = float(np.median(times))
    # The same layer once more on one thread (BLAS limited to 1), when that
    # stays within ~15 s of CPU time.
    one_thread = None
    if dt * threads <= 15.0:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                ssq = oracle.stats(data["X"], wl.xdtype)
                s = oracle.awq_scales(ssq, wl.T, wl.alpha, wl.lambda_rel)
                v = oracle.quant_values(data["W"], wl.wdtype, s, B, A)
                r = oracle.group_rtn(v, wl.bits, wl.group)
                oracle.pack_codes(r["q"], wl.bits)
                w_hat = oracle.dequant(r["q"], r["delta"], r["zero"], wl.group)
                oracle.project(data["X"], wl.xdtype, s, w_hat, B, A)
                one_thread = round((time.perf_counter() - t0) * 1e6, 1)
        except Exception:  # pragma: no cover
            one_thread = None
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    return {"value": round(dt * 1e6, 1), "unit": "us/layer", "cores": int(threads), "kind": "oracle",
            "sample": f"the full layer ({wl.T}x{wl.K}->{wl.M}) through the fp64 numpy oracle (stats, scales, "
                      f"quantize, pack, dequantize, projection), median of {len(times)} runs "
                      f"({sum(times):.1f} s of CPU work); cores = BLAS threads",
            "stages_us": {k: round(float(np.median(v)) * 1e6, 1) for k, v in stages.items()},
            "one_thread_us": one_thread,
            "cpu_model": cpu_model, "host_cpus": avail}


def _graph_time_us(calls, reps: int, warm: int) -> float:
    """Average µs of one call of ``calls`` (a Python function enqueuing a list
    of n calls), captured once in a HIP graph and replayed ``reps`` times."""
    import torch
    calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        n = calls()
    torch.cuda.synchronize()
    for _ in range(max(1, warm)):
        graph.replay()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record()
    for _ in range(reps):
        graph.replay()
    f1.record()
    torch.cuda.synchronize()
    return f0.elapsed_time(f1) / (reps * n) * 1e3


def bench_workload(wl, args, dev, with_cpu: bool) -> dict:
    """Time one workload: the whole layer (timed region), its stages (kernel
    stamps), and, where the workload has them, decode steps and per-prompt
    factors.  Returns a dict of results (µs, rates, fractions of peak)."""
    import numpy as np
    import torch
    from online_activation_aware_amd import synth, ttq

    log(f"workload {wl.key}: {wl.name}")
    data = synth.make_inputs(wl)

    def to_dev(a, dt):
        t = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) if dt == "bf16"
             else torch.from_numpy(np.ascontiguousarray(a)))
        return t.to(dev)

    X0, W0 = to_dev(data["X"], wl.xdtype), to_dev(data["W"], wl.wdtype)
    per_copy = X0.numel() * X0.element_size() + W0.numel() * W0.element_size()
    ncopy = max(2, min(64, math.ceil((args.min_rotation_mib << 20) / per_copy)))
    Xs = [X0] + [X0.clone() for _ in range(ncopy - 1)]
    Ws = [W0] + [W0.clone() for _ in range(ncopy - 1)]
    log(f"{ncopy} rotating input copies ({ncopy * per_copy / 2**20:.0f} MiB)")

    B = A = None
    B_h = A_h = None
    factors = None
    if wl.rank:
        # Per-prompt factors of W diag(s) on the GPU (randomized subspace
        # iteration, l = rank + 8 test vectors, q = 2 power iterations); the
        # layer below uses them, and they are timed on their own.
        ssq = torch.empty(wl.K, dtype=torch.float64, device=dev)
        ttq.ttq_stats(X0, ssq, ws=ttq.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group, wl.rank, device=dev))
        s0 = ttq.ttq_awq_scales(ssq, wl.T, wl.alpha, wl.lambda_rel)
        l_f, q_f = wl.rank + 8, 2
        om = torch.from_numpy(synth.test_vectors(l_f, wl.K, seed=0)).to(dev)
        B, A = ttq.ttq_lowrank_factors(W0, s0, om, wl.rank, q_f)
        torch.cuda.synchronize()
        B_h, A_h = B.cpu().numpy(), A.cpu().numpy()
        factors = time_factors(ttq, Ws, s0, om, wl, l_f, q_f, args)
        log(f"  factors   {factors['us']:8.2f} us  (l={l_f}, q={q_f}, {factors['passes_over_w']} passes over W)")

    st = ttq.linear_state(wl.T, wl.K, wl.M, wl.bits, wl.group, device=dev)
    ws = ttq.workspace(wl.T, wl.K, wl.M, wl.bits, wl.group, wl.rank, device=dev)
    Y = torch.empty((wl.T, wl.M), dtype=torch.float32, device=dev)

    def step(i, events=None):
        ttq.ttq_linear(Xs[i % ncopy], Ws[i % ncopy], wl.bits, wl.group, wl.alpha, wl.lambda_rel,
                       B=B, A=A, Y=Y, ws=ws, state=st, stage_events=events)

    # Clock settling before the warm-up: steps run back to back for
    # --settle-ms of wall time (untimed, reported as "settle").  On a GPU that
    # was idle the clocks take tens of milliseconds of sustained work to reach
    # their steady level; a handful of warm-up steps alone leaves the first
    # timed steps ~10% slow (c2: ~99 us/layer after 5 steps, ~90 once warm).
    settle_steps = 0
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(16):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"settled ({settle_steps} steps, {settle_ms:.0f} ms), warmup done ({args.warmup} steps)")

    # Timed region: K steps back to back, each ttq_linear called from
    # Python, nothing else on the stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms * 1e3:.1f} us/layer (wall {wall * 1e3 / args.steps * 1e3:.1f} us/step)")

    # Instrumented region: K more steps in which ttq_linear stamps HIP events
    # with its own kernels' start and end times on the launch stream
    # (hipExtLaunchKernel), one (start, stop) pair per stage.  The stamps cost
    # a few microseconds of launch latency per kernel, so this region is not
    # the one the layer time comes from; the kernel durations themselves are
    # exact.
    evs = [ttq.StageEvents() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per_step = [e.stage_ms() for e in evs]
    stage_ms = {k: sum(p[k] for p in per_step) / args.steps for k in ttq.LINEAR_STAGES}

    def pct(vals, q):
        v = sorted(vals)
        return v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
    if not wl.rank:
        stage_ms.pop("lowrank")

    alg = algorithmic_bytes(wl)
    flops = 2.0 * wl.T * wl.M * wl.K
    proj_us = stage_ms["projection"] * 1e3
    achieved = flops / (proj_us * 1e-6) / 1e12
    breakdown = {}
    for name, v in stage_ms.items():
        us = v * 1e3
        d = {"us": round(us, 2)}
        vals = [p[name] * 1e3 for p in per_step]
        d["p10_p50_p90_us"] = [round(pct(vals, q), 2) for q in (0.1, 0.5, 0.9)]
        if name in alg:
            d["alg_bytes"] = alg[name]
            d["gbs"] = round(alg[name] / (us * 1e-6) / 1e9, 1)
            d["hbm_frac"] = round(d["gbs"] / PEAK_HBM_GBS, 4)
        if name == "quantize" and wl.T >= 192 and wl.xdtype == "bf16":
            d["staged_bytes"] = wl.M * wl.K * 2     # dequantized weight written for the projection
        breakdown[name] = d
    breakdown["projection"]["tflops"] = round(achieved, 2)
    breakdown["projection"]["mfma_frac"] = round(achieved / PEAK_BF16_TFLOPS, 4)
    for name, d in breakdown.items():
        log(f"  {name:10s} {d['us']:8.2f} us" + (f"  {d['gbs']:8.1f} GB/s" if "gbs" in d else "")
            + (f"  {d['tflops']:8.1f} TFLOP/s" if "tflops" in d else ""))

    # Decode steps (workloads with decode tokens): ttq_qgemm on the prompt's
    # quantized state for T new tokens, over rotating copies of the state
    # (cold in the Infinity Cache).  One step per copy is captured in a HIP
    # graph, so that the figure is the kernels' and not the host's launch rate.
    decode = None
    if wl.decode_T:
        decode = {}
        sbytes = sum(st[k].numel() * st[k].element_size() for k in ("codes", "scale_f16", "zero_f16"))
        nst = max(2, min(64, math.ceil((args.min_rotation_mib << 20) / sbytes)))
        states = [{k: st[k].clone() for k in ("s", "codes", "scale_f16", "zero_f16")} for _ in range(nst)]
        wsd = ttq.workspace(max(wl.decode_T), wl.K, wl.M, wl.bits, wl.group, device=dev)
        for td in wl.decode_T:
            Xd = to_dev(data["X_decode"][td], wl.xdtype)
            Yd = torch.empty((td, wl.M), dtype=torch.float32, device=dev)

            def dsteps():
                for q in states:
                    ttq.ttq_qgemm(Xd, q["s"], q["codes"], q["scale_f16"], q["zero_f16"], wl.M, wl.bits,
                                  wl.group, Y=Yd, ws=wsd)
                return len(states)
            us = _graph_time_us(dsteps, max(1, math.ceil(args.steps / nst)), math.ceil(args.warmup / nst))
            b = sbytes + wl.K * 4 + td * wl.K * esize(wl.xdtype) + td * wl.M * 4
            decode[str(td)] = {"us": round(us, 2), "alg_bytes": b, "gbs": round(b / (us * 1e-6) / 1e9, 1),
                               "hbm_frac": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                               "flops": 2 * td * wl.M * wl.K}
            log(f"  decode T={td:<3d} {us:8.2f} us  {decode[str(td)]['gbs']:8.1f} GB/s "
                f"({nst} rotating state copies in one graph)")

        # One decode token for each of P prompts (each with its own quantized
        # state) in one ttq_qgemm_batched launch, over rotating groups.
        P = 8
        ngr = max(2, min(8, math.ceil((args.min_rotation_mib << 20) / (P * sbytes))))
        groups = [{k: torch.stack([st[k].clone() for _ in range(P)]) for k in ("s", "codes", "scale_f16", "zero_f16")}
                  for _ in range(ngr)]
        Xb = to_dev(data["X_decode"][1], wl.xdtype).unsqueeze(0).repeat(P, 1, 1).contiguous()
        Yb = torch.empty((P, 1, wl.M), dtype=torch.float32, device=dev)

        def bsteps():
            for g in groups:
                ttq.ttq_qgemm_batched(Xb, g["s"], g["codes"], g["scale_f16"], g["zero_f16"], wl.M, wl.bits,
                                      wl.group, Y=Yb)
            return len(groups)
        us = _graph_time_us(bsteps, max(1, math.ceil(args.steps / ngr)), 1)
        b = P * (sbytes + wl.K * 4 + wl.K * esize(wl.xdtype) + wl.M * 4)
        decode["batched_P8_T1"] = {"us": round(us, 2), "prompts": P, "alg_bytes": b,
                                   "gbs": round(b / (us * 1e-6) / 1e9, 1),
                                   "hbm_frac": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                   "tokens_per_s": round(P / (us * 1e-6), 1)}
        log(f"  decode P={P} prompts x T=1 {us:8.2f} us  {decode['batched_P8_T1']['gbs']:8.1f} GB/s "
            f"({ngr} rotating groups)")
        del states, groups

    cpu = None
    if with_cpu:
        log("timing the CPU oracle on the same layer ...")
        cpu = cpu_baseline(wl, data, B_h, A_h)
        log(f"  oracle: {cpu['value'] / 1e6:.2f} s/layer on {cpu['cores']} BLAS threads")

    out = {"us_per_layer": round(ms * 1e3, 3), "workload": wl.name,
           "config": {"workload": wl.name, "T": wl.T, "K": wl.K, "M": wl.M, "bits": wl.bits, "group": wl.group,
                      "alpha": wl.alpha, "lambda_rel": wl.lambda_rel, "rank": wl.rank, "x_dtype": wl.xdtype,
                      "w_dtype": wl.wdtype, "y_dtype": "f32",
                      "cache": f"{ncopy} rotating copies of X and W ({ncopy * per_copy / 2**20:.0f} MiB)"},
           "stages": breakdown, "decode": decode, "factors": factors, "cpu_baseline": cpu,
           "projection_flops": flops, "projection_us": proj_us,
           "settle": {"steps": settle_steps, "ms": round(settle_ms, 1)}}
    del Xs, Ws, X0, W0, st, ws, Y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    # Untimed steps for this many ms of wall time before the warm-up steps of
    # each workload, so that the clocks have settled whatever --warmup is.
    ap.add_argument("--settle-ms", type=float, default=150.0)
    ap.add_argument("--workload", default="all",
                    help="all (default: c2 as the headline, then c1, c3, c4, c5) or one of c1..c5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-rotation-mib", type=int, default=1024)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this size (for HBM counter scaling)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the path needs no cross-GPU exchange and each GPU runs it independently.", file=sys.stderr)
        return 2

    import torch
    from online_activation_aware_amd import synth, ttq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 3 times")
        return 0

    ttq.lib()  # fail loudly if the HIP library is missing
    keys = ["c2", "c1", "c3", "c4", "c5"] if args.workload == "all" else [args.workload]
    results = {}
    for i, key in enumerate(keys):
        results[key] = bench_workload(synth.workload(key), args, dev, with_cpu=(i == 0 and not args.no_cpu_baseline))
    head = results[keys[0]]

    proj_us = head["projection_us"]
    achieved = head["projection_flops"] / (proj_us * 1e-6) / 1e12
    h = kernel_source_hash()
    tr = MEASURED_TRAFFIC.get(h)
    traffic = tr["fetch_bytes"] + tr["write_bytes"] if tr and tr["workload"] == keys[0] else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "k_gemm_bf16 (Y = X W~^T on the dequantized weight; bf16 MFMA 16x16x32, "
                          "fp32 accumulate, buffer->LDS DMA)",
                "flops_per_launch": head["projection_flops"], "avg_launch_us": round(proj_us, 2),
                "traffic_detail": (None if traffic is None else
                                   {"fetch_bytes": tr["fetch_bytes"], "write_bytes": tr["write_bytes"],
                                    "source": "stored: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE taken on this "
                                              "kernel source (hash " + h + "), not measured in this run",
                                    "counters": "FETCH_SIZE x2.0, WRITE_SIZE x1.0 (1 GiB copy calibration)"}),
                "timing": "kernel start/end stamped into HIP events by ttq_linear on its stream "
                          f"(hipExtLaunchKernel), averaged over {args.steps} instrumented steps"}

    def summary(r):
        d = {"us_per_layer": r["us_per_layer"], "config": r["config"], "stages": r["stages"],
             "settle": r["settle"]}
        if r["decode"]:
            d["decode"] = r["decode"]
        if r["factors"]:
            d["factors"] = r["factors"]
        return d

    out = {
        "metric": METRIC,
        "value": head["us_per_layer"],
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": dict(head["settle"], note="untimed steps run for --settle-ms of wall time before the "
                       "warm-up steps, so the clocks have settled whatever --warmup is"),
        "ms_per_step": round(head["us_per_layer"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": roofline,
        "cpu_baseline": head["cpu_baseline"],
        "stages": head["stages"],
        "decode": head["decode"],
        "factors": head["factors"],
        "workloads": {k: summary(r) for k, r in results.items()},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
