#!/usr/bin/env python3
"""Benchmark of gather_qmm on one MI355X.

Workload (ml-explore/mlx issue 4339, "Kernel microbenchmark"): T=2048 tokens,
top-8 of E=64 experts, K=2048, N=768, x ~ N(0,1) bf16 [2048, 8, 1, 2048],
W ~ N(0,1) bf16 [64, 768, 2048] affine-quantised to 4 bits in groups of 64
(offline, before timing), indices uniform in [0, 64).  Beside it, as on the
page: the same call with pre-sorted indices and the equal-FLOPs dense
quantised matmul x [16384, 2048] x one quantised [768, 2048].

One step = one mq_gather_qmm call: routing (histogram, scan, stable scatter)
and the per-group row sums of x, then the gathered grouped GEMM with its fused
unpermuting store.  Inputs are resident in HBM before timing starts; the same
buffers are reused every step, as in the page's benchmark loop.

Prints ONE JSON line.  Timing: before each variant, back-to-back calls for at
least 0.3 s (the GPU's engine clock rises from ~1.9 GHz to ~2.3 GHz over the
first ~100 ms of sustained load), then W warm-up steps, then exactly K steps
between two torch.cuda.synchronize() calls (wall clock, nothing recorded in
between); then K more calls with HIP events recorded on the launch stream
around each, and the same for K launches of the GEMM kernel alone
(mq_gather_qmm_routed on a workspace holding the routing) for the roofline of
the dominant kernel.

Before any timing, the cpu_baseline leg runs the CPU oracle on a bounded
sample of the same workload (the first tokens, ~10 s with all host threads
and ~10 s with one), which gives the oracle's throughput, and compares the
sampled outputs with the GPU's output of the timed call element by element
(the tolerance gate of the parity tests); a failure ends the run with an
error instead of a number.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6        # MI355X dense bf16 MFMA (256 CU x 4 SIMD x 1024 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0
METRIC = "gather_qmm TFLOPs + % bf16 MFMA peak vs equal-FLOPs dense qmm, 1×MI355X"


def _progress(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def recorded_traffic(profile: str, key: str = "traffic_bytes_per_launch",
                     sources=("quantized_moe_grouped_amd/csrc/gemm.hip",)):
    """HBM bytes as last measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy kernel), read from the committed profile
    summary (`key: value` lines); None if a kernel source it depends on changed
    since (each source's `<file name>_sha256_16: ...` line must match)."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        shas = {os.path.basename(src): hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]
                for src in sources}
    except OSError:
        return None
    vals = dict(l.strip().split(": ", 1) for l in text.splitlines() if l.startswith("    ") and ": " in l)
    for name, sha in shas.items():
        if vals.get(f"{name}_sha256_16") != sha:
            return None
    return int(vals[key]) if key in vals else None


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def _oracle_timed(oracle, case, wq, s, b, tokens: int, seconds: float):
    """The oracle's gather_qmm on the first `tokens` tokens, called until
    `seconds` have passed (at least once); returns (TFLOP/s, calls, seconds,
    the last output)."""
    import numpy as np
    x = np.ascontiguousarray(case.x[:tokens])
    idx = np.ascontiguousarray(case.idx[:tokens])
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = oracle.gather_qmm(x, wq, s, b, idx, case.group_size, case.bits)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return 2.0 * tokens * case.A * case.K * case.N * reps / dt / 1e12, reps, dt, ref


def _c_oracle_timed(co, case, wq, s, b, tokens: int, seconds: float):
    """The fp32 C oracle's gather_qmm on the first `tokens` tokens, called until
    `seconds` have passed; returns (TFLOP/s, calls, seconds, last output)."""
    import numpy as np
    x = np.ascontiguousarray(case.x[:tokens])
    idx = np.ascontiguousarray(case.idx[:tokens])
    reps = 0
    t0 = time.perf_counter()
    while True:
        out = co.gather_qmm(x, wq, s, b, idx, case.group_size, case.bits)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return 2.0 * tokens * case.A * case.K * case.N * reps / dt / 1e12, reps, dt, out


def c_oracle_baseline(case, gpu_out, sample_tokens: int, seconds: float):
    """The fp32 C oracle (plain loop nests, OpenMP over output rows) on the
    GPU machine's host: all threads and one thread, quantise / route / product
    timed apart, and the timed call's GPU output checked against its result."""
    import numpy as np
    from oracle import c_oracle
    co = c_oracle.Oracle()
    t0 = time.perf_counter()
    wq, s, b = co.quantize(case.w, case.group_size, case.bits)
    t_quant = time.perf_counter() - t0
    t0 = time.perf_counter()
    co.route(case.idx, case.E)
    t_route = time.perf_counter() - t0
    threads = co.threads()
    sample_tokens = min(sample_tokens, case.T)
    value, reps, dt, out = _c_oracle_timed(co, case, wq, s, b, sample_tokens, seconds)
    try:
        co.threads(1)
        one_tokens = max(1, sample_tokens // 16)
        v1, reps1, dt1, _ = _c_oracle_timed(co, case, wq, s, b, one_tokens, seconds)
    finally:
        co.threads(threads)
    ref = out.reshape(-1, case.N).astype(np.float64)
    got = gpu_out[:ref.shape[0]]
    worst = float((np.abs(got - ref) / (1e-2 * np.maximum(1.0, np.abs(ref)))).max())
    return {"value": value, "unit": "TFLOPs", "cores": threads, "kind": "oracle (fp32 C)",
            "seconds": round(dt, 3), "calls": reps,
            "sample": f"{reps} calls on {sample_tokens} of {case.T} tokens ({sample_tokens * case.A} "
                      f"routed rows each), fp32 C oracle incl. dequantisation of all {case.E} experts",
            "single_thread": {"value": v1, "cores": 1, "seconds": round(dt1, 3), "calls": reps1,
                              "sample": f"{reps1} calls on {one_tokens} tokens"},
            "split_seconds": {"quantize_all_experts": round(t_quant, 3),
                              "route_all_pairs": round(t_route, 4),
                              "gather_qmm_per_call_on_sample": round(dt / reps, 3)},
            "gpu_output_worst_err_over_gate": round(worst, 4)}


def cpu_baseline(case, gpu_out, sample_tokens: int, seconds: float):
    """The oracle, as it stands, on the first `sample_tokens` tokens with all
    host threads and on 1/8 of them with one thread, each repeated until
    `seconds` have passed; its output for the sampled tokens is compared with
    the GPU's output of the timed call (gpu_out: fp64 [T*A, N])."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    wq, s, b = oracle.quantize(case.w, case.group_size, case.bits)      # offline: not in the rate
    t_quant = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.route(case.idx, case.E)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.dequantize(wq, s, b, case.group_size, case.bits)
    t_deq = time.perf_counter() - t0
    sample_tokens = min(sample_tokens, case.T)
    value, reps, dt, ref = _oracle_timed(oracle, case, wq, s, b, sample_tokens, seconds)
    cores = _blas_threads()
    one_tokens = max(1, sample_tokens // 8)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            v1, reps1, dt1, _ = _oracle_timed(oracle, case, wq, s, b, one_tokens, seconds)
        one = {"value": v1, "cores": 1, "seconds": round(dt1, 3), "calls": reps1,
               "sample": f"{reps1} calls on {one_tokens} tokens"}
    except ImportError:
        one = None
    # parity of the timed call's output on the sampled rows (the gate of the
    # parity tests: |err| <= 1e-2 max(1, |ref|) per element, relative
    # Frobenius error <= 4e-3)
    ref = ref.reshape(-1, case.N)
    got = gpu_out[:ref.shape[0]]
    err = np.abs(got - ref)
    worst = float((err / (1e-2 * np.maximum(1.0, np.abs(ref)))).max())
    fro = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    # distance of each bf16 output from the oracle's value rounded to bf16
    # (nearest even), in units in the last place: 0 wherever fp32
    # accumulation left the rounding unchanged
    def bf16_key(v):
        b = (np.asarray(v, np.float32).view(np.uint32) + np.uint32(0x7FFF) +
             ((np.asarray(v, np.float32).view(np.uint32) >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        b = b.astype(np.int64)
        return np.where(b & 0x8000, 0x8000 - b, b)      # monotone in the value
    ulps = np.abs(bf16_key(got) - bf16_key(ref))
    big = np.abs(ref) >= 2.0 ** -4          # away from zero, where a ulp count means something
    parity = {"outputs_checked": int(ref.size), "worst_err_over_gate": round(worst, 4),
              "rel_frobenius": fro,
              "frac_equal_to_rounded_oracle": float((ulps == 0).mean()),
              "max_ulps_where_abs_ref_ge_1/16": int(ulps[big].max()) if big.any() else 0,
              "pass": bool(worst <= 1.0 and fro <= 4e-3)}
    return {"value": value, "unit": "TFLOPs", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3), "calls": reps,
            "sample": f"{reps} calls on {sample_tokens} of {case.T} tokens ({sample_tokens * case.A} "
                      f"routed rows each), fp64 numpy oracle incl. dequantisation of all {case.E} experts",
            "single_thread": one,
            "split_seconds": {"quantize_all_experts": round(t_quant, 3),
                              "route_all_pairs": round(t_route, 4),
                              "dequantize_all_experts": round(t_deq, 3),
                              "gather_qmm_per_call_on_sample": round(dt / reps, 3),
                              "note": "the oracle's gather_qmm dequantises every expert on each "
                                      "call, then multiplies the sampled rows in fp64"}}, parity


def small_m_bench(mq, torch, np, workloads, dev, reps: int, graphs: bool = True):
    """Batched-decode shapes (lablup/mlxcel issue 725, "The gap"): dense
    quantised matmuls with B <= 8 rows and a top-8 MoE decode step.  Enough
    weight copies are cycled that their total exceeds the 256 MB Infinity
    Cache, so each call streams its weight from HBM; the figure is algorithmic
    bytes (codes + scales + biases read once, x, out) over the event time."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed(fns):
        # These calls take a few microseconds, less than the host needs to
        # submit one, so they are captured once into a HIP graph (one launch
        # per weight copy, round robin) and the graph is replayed; the time per
        # call is the replay time over the number of calls.  (graphs=False:
        # direct calls, for counter runs of a profiler that sees no graph
        # launches; the time then includes the host's submission gaps.)
        for f in fns:
            f()
        torch.cuda.synchronize()
        if not graphs:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                for f in fns:
                    f()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / (reps * len(fns))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for f in fns:
                    f()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * len(fns))

    res = []
    for (N, K, bits, gs) in [(14336, 4096, 4, 64), (4096, 14336, 4, 64), (14336, 4096, 8, 32)]:
        _, w = workloads.small_m_dense(1, N, K, seed=7)
        wq0, s0, b0 = mq.mq_quantize(to_bf16(w), gs, bits)
        wbytes = wq0.numel() * 4 + s0.numel() * 4
        copies = max(2, int(np.ceil(600e6 / wbytes)))
        ws = [(wq0.clone(), s0.clone(), b0.clone()) for _ in range(copies)]
        for B in (1, 2, 4, 8):
            x = to_bf16(workloads.small_m_dense(B, N, K, seed=B)[0])
            out = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty(max(mq.mq_qmm_workspace(B, K, gs), 256), dtype=torch.uint8, device=dev)
            fns = [lambda q=q: mq.mq_qmm(x, q[0], q[1], q[2], True, gs, bits, out=out, workspace=wsp)
                   for q in ws]
            ms = timed(fns)
            byt = wbytes + B * K * 2 + B * N * 2
            res.append({"shape": f"dense B={B} N={N} K={K} {bits}-bit gs{gs}", "us": round(ms * 1e3, 2),
                        "GB/s": round(byt / (ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        del ws
    case = workloads.moe_decode(0)
    wq0, s0, b0 = mq.mq_quantize(to_bf16(case.w), 64, 4)
    per_expert = (wq0[0].numel() + s0[0].numel()) * 4
    copies = max(2, int(np.ceil(600e6 / (per_expert * case.E))))
    ws = [(wq0.clone(), s0.clone(), b0.clone()) for _ in range(copies)]
    x = to_bf16(case.x)
    idx = torch.from_numpy(case.idx).to(dev)
    out = torch.empty((case.T, case.A, 1, case.N), dtype=torch.bfloat16, device=dev)
    L = mq.mq_gather_qmm_workspace(case.T, case.A, 1, case.K, case.N, case.E, 64, 4)
    wsp = torch.empty(L.total, dtype=torch.uint8, device=dev)
    fns = [lambda q=q: mq.mq_gather_qmm(x, q[0], q[1], q[2], idx, True, 64, 4, False, out=out,
                                        workspace=wsp) for q in ws]
    ms = timed(fns)
    touched = int(np.unique(case.idx).size)
    byt = touched * per_expert + case.T * case.A * (case.K + case.N) * 2
    res.append({"shape": f"MoE decode T=4 top-8 E=128 K=2048 N=768 4-bit gs64 ({touched} experts touched)",
                "us": round(ms * 1e3, 2), "GB/s": round(byt / (ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
    return res


def _warm_then_time(torch, fns, steps, warm_s=0.3):
    """Run the list of calls back to back for ~warm_s seconds (engine clock),
    then time `steps` rounds of it with HIP events around each call; returns
    the per-call median times (ms)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for f in fns:
            f()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in fns] for _ in range(steps)]
    for row in ev:
        for (a, b), f in zip(row, fns):
            a.record(stream)
            f()
            b.record(stream)
    torch.cuda.synchronize()
    import statistics
    return [statistics.median(row[i][0].elapsed_time(row[i][1]) for row in ev) for i in range(len(fns))]


def _touched_bytes(case, K, N, bits, gs):
    """codes + scales + biases of the experts the routing touches (once each)"""
    import numpy as np
    touched = int(np.unique(case.idx).size)
    return touched * N * (K * bits // 8 + 2 * 2 * (K // gs))


def short_run_sweep_bench(mq, torch, np, workloads, dev, steps):
    """E=256, top-8, K=2048 -> N=512 up, then 512 -> 2048 down on the up's
    output (ml-explore/mlx PR 4023, "The change": its decode/prefill sweep of
    chained up and down projections over short runs), exactly r rows per
    expert.  One strip = mq_gather_qmm(up) then mq_gather_qmm(down), each with
    its own routing launch."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    res = []
    wu = wd = None
    for r in (4, 8, 16, 32, 64, 128):
        case = workloads.short_run_sweep(r, seed=0)
        T, A, E = case.T, case.A, case.E
        if wu is None:                                 # the weights do not depend on r
            wu = mq.mq_quantize(to_bf16(case.w), 64, 4)
            wd = mq.mq_quantize(to_bf16(case.w_down), 64, 4)
        x = to_bf16(case.x)
        idx = torch.from_numpy(case.idx).to(dev)
        h = torch.empty((T, A, 1, 512), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, A, 1, 2048), dtype=torch.bfloat16, device=dev)
        Lu = mq.mq_gather_qmm_workspace(T, A, 1, 2048, 512, E, 64, 4)
        Ld = mq.mq_gather_qmm_workspace(T, A, 1, 512, 2048, E, 64, 4)
        ws = torch.empty(max(Lu.total, Ld.total), dtype=torch.uint8, device=dev)
        up = lambda: mq.mq_gather_qmm(x, *wu, idx, True, 64, 4, False, out=h, workspace=ws)
        down = lambda: mq.mq_gather_qmm(h, *wd, idx, True, 64, 4, False, out=y, workspace=ws)
        t_up, t_down = _warm_then_time(torch, [up, down], steps)
        n = T * A
        flops = 2.0 * n * 2048 * 512
        b_up = _touched_bytes(case, 2048, 512, 4, 64) + n * (2048 + 512) * 2
        b_down = _touched_bytes(case, 512, 2048, 4, 64) + n * (512 + 2048) * 2
        res.append({"rows_per_expert": r, "T": T, "strip_us": round((t_up + t_down) * 1e3, 2),
                    "up_us": round(t_up * 1e3, 2), "down_us": round(t_down * 1e3, 2),
                    "up_TFLOPs": round(flops / (t_up * 1e-3) / 1e12, 2),
                    "down_TFLOPs": round(flops / (t_down * 1e-3) / 1e12, 2),
                    "mfma_peak_frac": round(2 * flops / ((t_up + t_down) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "hbm_frac": round((b_up + b_down) / ((t_up + t_down) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
        del ws, x, h, y
    return res


def glu_bench(mq, torch, np, workloads, dev, steps):
    """The Mixtral-shaped gate and up projections (E=8, top-2, T=2048, K=4096
    -> F=14336, Zipf(1.2) routing, W ~ N(0, 0.02)) with SiLU: one fused
    mq_gather_qmm_glu call, against two mq_gather_qmm calls followed by the
    activation and product as separate elementwise passes."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    g = workloads.mixtral_ffn(0, 1.2, "up")
    T, A, E, K, F = g.T, g.A, g.E, g.K, g.N
    up_w = workloads.gather_case("mixtral-up2", 8, 1, E, K, F, seed=77, w_std=0.02).w
    gate = mq.mq_quantize(to_bf16(g.w), 64, 4)
    up = mq.mq_quantize(to_bf16(up_w), 64, 4)
    x = to_bf16(g.x)
    idx = torch.from_numpy(g.idx).to(dev)
    ws = torch.empty(mq.mq_gather_qmm_workspace(T, A, 1, K, F, E, 64, 4).total, dtype=torch.uint8,
                     device=dev)
    h = torch.empty((T, A, 1, F), dtype=torch.bfloat16, device=dev)
    gb, ub, h2 = torch.empty_like(h), torch.empty_like(h), torch.empty_like(h)
    fused = lambda: mq.mq_gather_qmm_glu(x, gate, up, idx, mq.ACT_SILU, out=h, workspace=ws)

    def separate():
        mq.mq_gather_qmm(x, *gate, idx, out=gb, workspace=ws)
        mq.mq_gather_qmm(x, *up, idx, out=ub, workspace=ws)
        torch.mul(torch.nn.functional.silu(gb), ub, out=h2)

    def shared_routing():
        mq.mq_gather_route(idx, E, 1, workspace=ws, K=K)
        mq.mq_gather_sums(x, A, E, ws)
        mq.mq_gather_qmm_routed(x, *gate, A, ws, out=gb)
        mq.mq_gather_qmm_routed(x, *up, A, ws, out=ub)
    tf, ts, tr = _warm_then_time(torch, [fused, separate, shared_routing], steps)
    flops = 2 * 2.0 * T * A * K * F
    return {"shape": "E=8 top-2 T=2048, gate and up K=4096 -> F=14336, 4-bit gs64, SiLU",
            "fused_us": round(tf * 1e3, 2), "fused_TFLOPs": round(flops / (tf * 1e-3) / 1e12, 2),
            "separate_us": round(ts * 1e3, 2),
            "shared_routing_two_projections_us": round(tr * 1e3, 2),
            "fused_vs_separate": round(ts / tf, 4)}


def gather_nn_bench(mq, torch, np, workloads, dev, steps):
    """The untransposed product (ml-explore/mlx PR 4023, the coverage reply:
    the backward pass's orientation, timed there at E=4, K=D=512, B=1024):
    1024 routed rows (top-1, uniform over 4 experts), one quantised stack
    [4, 512, 512] (4-bit gs64) applied as x @ w_hat[e]; beside it the forward
    call x @ w_hat[e]^T on the same stack and an equal-FLOPs dense control
    (one [512, 512] weight, transpose=0)."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    case = workloads.gather_case("nn-E4-K512-B1024", 1024, 1, 4, 512, 512, seed=0)
    T, A, E, K, N = case.T, case.A, case.E, case.K, case.N
    x = to_bf16(case.x)
    idx = torch.from_numpy(case.idx).to(dev)
    wq, sc, bs = mq.mq_quantize(to_bf16(case.w), 64, 4)          # stored [4, 512, 512]
    out = torch.empty((T, A, 1, N), dtype=torch.bfloat16, device=dev)
    outf = torch.empty_like(out)
    ws = torch.empty(mq.mq_gather_qmm_workspace(T, A, 1, K, N, E, 64, 4).total, dtype=torch.uint8,
                     device=dev)
    xd = x.reshape(T * A, K)
    outd = torch.empty((T * A, N), dtype=torch.bfloat16, device=dev)
    nn = lambda: mq.mq_gather_qmm(x, wq, sc, bs, idx, False, 64, 4, False, out=out, workspace=ws)
    fwd = lambda: mq.mq_gather_qmm(x, wq, sc, bs, idx, True, 64, 4, False, out=outf, workspace=ws)
    dense = lambda: mq.mq_qmm(xd, wq[0], sc[0], bs[0], False, 64, 4, out=outd)
    t, tf, td = _warm_then_time(torch, [nn, fwd, dense], steps)
    flops = 2.0 * T * A * K * N
    return {"shape": "E=4, 1024 routed rows (top-1), K=D=512, 4-bit gs64, stored [4, 512, 512], "
                     "transpose=0", "us": round(t * 1e3, 2), "TFLOPs": round(flops / (t * 1e-3) / 1e12, 2),
            "forward_transpose1_us": round(tf * 1e3, 2),
            "dense_control_us": round(td * 1e3, 2), "gather_vs_dense": round(td / t, 4)}


def gather_mm_bench(mq, torch, np, workloads, dev, steps):
    """The unquantised gather (ml-explore/mlx issue 4339, the bf16 MoE gather
    path) at the prefill shape: the same x and routing, the bf16 expert
    weights the quantised case starts from [64, 768, 2048], next to an
    equal-FLOPs dense control (one bf16 [768, 2048] weight, every index 0)."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    case = workloads.prefill_microbench(0)
    T, A, E, K, N = case.T, case.A, case.E, case.K, case.N
    x = to_bf16(case.x)
    w = to_bf16(case.w)
    idx = torch.from_numpy(case.idx).to(dev)
    out = torch.empty((T, A, 1, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mq.mq_gather_mm_workspace(T, A, 1, K, N, E).total, dtype=torch.uint8, device=dev)
    w1 = w[:1].contiguous()
    idx0 = torch.zeros_like(idx)
    ws1 = torch.empty(mq.mq_gather_mm_workspace(T, A, 1, K, N, 1).total, dtype=torch.uint8, device=dev)
    out1 = torch.empty_like(out)
    call = lambda: mq.mq_gather_mm(x, w, idx, True, False, out=out, workspace=ws)
    dense = lambda: mq.mq_gather_mm(x, w1, idx0, True, False, out=out1, workspace=ws1)
    t, td = _warm_then_time(torch, [call, dense], steps)
    flops = 2.0 * T * A * K * N
    touched = int(np.unique(case.idx).size)
    byt = touched * N * K * 2 + T * A * (K + N) * 2
    return {"shape": "T=2048 A=8 E=64 K=2048 N=768, bf16 weights [64, 768, 2048], uniform routing",
            "us": round(t * 1e3, 2), "TFLOPs": round(flops / (t * 1e-3) / 1e12, 2),
            "mfma_peak_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(byt / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": byt,
            "dense_control_us": round(td * 1e3, 2),
            "dense_control_TFLOPs": round(flops / (td * 1e-3) / 1e12, 2),
            "gather_vs_dense": round(td / t, 4)}


def gather_mx_bench(mq, torch, np, workloads, dev, steps, bits=4):
    """An MX mode (the pages' mxfp4 / mxfp8, read as OCP MX v1.0) at the
    prefill shape: the same x, routing and bf16 weights as the affine case,
    quantised on the device to E2M1 (bits 4) or E4M3 (bits 8) codes with one
    E8M0 exponent per 32 weights, next to an equal-FLOPs dense control (one
    [768, 2048] weight, every index 0)."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    case = workloads.prefill_microbench(0)
    T, A, E, K, N = case.T, case.A, case.E, case.K, case.N
    x = to_bf16(case.x)
    wq, sc = mq.mq_quantize_mx(to_bf16(case.w), bits)
    idx = torch.from_numpy(case.idx).to(dev)
    out = torch.empty((T, A, 1, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mq.mq_gather_mm_workspace(T, A, 1, K, N, E).total, dtype=torch.uint8, device=dev)
    wq1, sc1 = wq[:1].contiguous(), sc[:1].contiguous()
    idx0 = torch.zeros_like(idx)
    ws1 = torch.empty(mq.mq_gather_mm_workspace(T, A, 1, K, N, 1).total, dtype=torch.uint8, device=dev)
    out1 = torch.empty_like(out)
    call = lambda: mq.mq_gather_qmm_mx(x, wq, sc, idx, True, False, out=out, workspace=ws, bits=bits)
    dense = lambda: mq.mq_gather_qmm_mx(x, wq1, sc1, idx0, True, False, out=out1, workspace=ws1,
                                        bits=bits)
    t, td = _warm_then_time(torch, [call, dense], steps)
    flops = 2.0 * T * A * K * N
    touched = int(np.unique(case.idx).size)
    byt = touched * N * (K * bits // 8 + K // 32) + T * A * (K + N) * 2
    fmt = "MXFP4 weights (E2M1" if bits == 4 else "MXFP8 weights (E4M3"
    return {"shape": f"T=2048 A=8 E=64 K=2048 N=768, {fmt}, E8M0 per 32), uniform routing",
            "us": round(t * 1e3, 2), "TFLOPs": round(flops / (t * 1e-3) / 1e12, 2),
            "mfma_peak_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(byt / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": byt,
            "dense_control_us": round(td * 1e3, 2),
            "dense_control_TFLOPs": round(flops / (td * 1e-3) / 1e12, 2),
            "gather_vs_dense": round(td / t, 4)}


def gather_nv_bench(mq, torch, np, workloads, dev, steps):
    """The NVFP4 mode (the pages' nvfp4, read as NVIDIA's format) at the
    prefill shape: E2M1 codes, an E4M3 scale per 16 weights and an fp32 scale
    per expert, quantised on the device, next to the equal-FLOPs dense control."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    case = workloads.prefill_microbench(0)
    T, A, E, K, N = case.T, case.A, case.E, case.K, case.N
    x = to_bf16(case.x)
    wq, sc, g = mq.mq_quantize_nv(to_bf16(case.w))
    idx = torch.from_numpy(case.idx).to(dev)
    out = torch.empty((T, A, 1, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mq.mq_gather_mm_workspace(T, A, 1, K, N, E).total, dtype=torch.uint8, device=dev)
    wq1, sc1, g1 = wq[:1].contiguous(), sc[:1].contiguous(), g[:1].contiguous()
    idx0 = torch.zeros_like(idx)
    ws1 = torch.empty(mq.mq_gather_mm_workspace(T, A, 1, K, N, 1).total, dtype=torch.uint8, device=dev)
    out1 = torch.empty_like(out)
    call = lambda: mq.mq_gather_qmm_nv(x, wq, sc, g, idx, True, False, out=out, workspace=ws)
    dense = lambda: mq.mq_gather_qmm_nv(x, wq1, sc1, g1, idx0, True, False, out=out1, workspace=ws1)
    t, td = _warm_then_time(torch, [call, dense], steps)
    flops = 2.0 * T * A * K * N
    touched = int(np.unique(case.idx).size)
    byt = touched * (N * (K // 2 + K // 16) + 4) + T * A * (K + N) * 2
    return {"shape": "T=2048 A=8 E=64 K=2048 N=768, NVFP4 weights (E2M1, E4M3 per 16, fp32 per expert), "
                     "uniform routing",
            "us": round(t * 1e3, 2), "TFLOPs": round(flops / (t * 1e-3) / 1e12, 2),
            "mfma_peak_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(byt / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": byt,
            "dense_control_us": round(td * 1e3, 2),
            "dense_control_TFLOPs": round(flops / (td * 1e-3) / 1e12, 2),
            "gather_vs_dense": round(td / t, 4)}


def mixtral_bench(mq, torch, np, workloads, dev, steps):
    """E=8, top-2, T=2048; up K=4096 -> N=14336 and down K=14336 -> N=4096,
    4-bit gs64, W ~ N(0, 0.02), Zipf(1.2) routing (lablup/mlxcel issue 629's
    model shape).  The gate projection has the up projection's shape."""
    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    res = {}
    for proj in ("up", "down"):
        case = workloads.mixtral_ffn(0, 1.2, proj)
        T, A, E, K, N = case.T, case.A, case.E, case.K, case.N
        wq = mq.mq_quantize(to_bf16(case.w), 64, 4)
        x = to_bf16(case.x)
        idx = torch.from_numpy(case.idx).to(dev)
        out = torch.empty((T, A, 1, N), dtype=torch.bfloat16, device=dev)
        L = mq.mq_gather_qmm_workspace(T, A, 1, K, N, E, 64, 4)
        ws = torch.empty(L.total, dtype=torch.uint8, device=dev)
        call = lambda: mq.mq_gather_qmm(x, *wq, idx, True, 64, 4, False, out=out, workspace=ws)
        (t,) = _warm_then_time(torch, [call], steps)
        flops = 2.0 * T * A * K * N
        byt = _touched_bytes(case, K, N, 4, 64) + T * A * (K + N) * 2
        counts = np.bincount(case.idx.reshape(-1), minlength=E)
        res[proj] = {"K": K, "N": N, "us": round(t * 1e3, 1),
                     "TFLOPs": round(flops / (t * 1e-3) / 1e12, 2),
                     "mfma_peak_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "hbm_frac": round(byt / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "rows_per_expert": counts.tolist()}
        del wq, x, out, ws
    return res


def _probe_lib():
    """ctypes handle of the calibration probes (libmq_probe.so, include/mq_probe.h)."""
    import ctypes
    path = os.path.join(ROOT, "quantized_moe_grouped_amd", "libmq_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m quantized_moe_grouped_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mq_probe_stream.restype = ctypes.c_int
    lib.mq_probe_stream.argtypes = [P, I64, P, I32, P]
    lib.mq_probe_mfma.restype = ctypes.c_int
    lib.mq_probe_mfma.argtypes = [I32, P, I32, P]
    return lib


def measured_peaks(mq, torch, dev):
    """What this GPU delivers, from the library's calibration probes: HBM read
    bandwidth (one pass over 2 GiB, 16-byte loads, 2048 workgroups) and the
    dense bf16 MFMA rate (512 workgroups x 4 waves of register-only
    16x16x32 MFMAs), each the median of 10 timed runs after ~0.2 s of runs."""
    import statistics
    buf = torch.empty(1 << 29, dtype=torch.int32, device=dev).fill_(7)
    sink = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    iters = 16384
    fsink = torch.empty(512 * 256, dtype=torch.float32, device=dev)
    lib = _probe_lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run(status):
        if status != 0:
            raise RuntimeError(f"calibration probe failed: {mq.mq_status_str(status)}")
    calls = {"stream": lambda: run(lib.mq_probe_stream(buf.data_ptr(), buf.numel() * 4,
                                                       sink.data_ptr(), 2048, stream)),
             "mfma": lambda: run(lib.mq_probe_mfma(iters, fsink.data_ptr(), 512, stream))}
    res = {}
    for name, f in calls.items():
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            f()
            torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        res[name] = statistics.median(ts)
    del buf
    return {"hbm_read_GBs": round(buf_bytes(1 << 29, 4) / res["stream"] / 1e9, 1),
            "mfma_bf16_TFLOPs": round(512 * 4 * iters * 8 * 16384 / res["mfma"] / 1e12, 1),
            "how": "mq_probe_stream over 2 GiB / mq_probe_mfma (random bf16 operands), median of 10 after warm-up"}


def buf_bytes(n, size):
    return n * size


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed calls before each timed variant, after >= 0.3 s of calls that "
                         "let the engine clock settle at its sustained-load level")
    ap.add_argument("--cpu-sample-tokens", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle on the sample until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-small-m", action="store_true", help="skip the batched-decode shapes")
    ap.add_argument("--no-sweeps", action="store_true",
                    help="skip the short-run sweep (E=256) and the Mixtral-shape projections")
    ap.add_argument("--no-graphs", action="store_true",
                    help="launch the batched-decode calls directly instead of replaying HIP graphs "
                         "(for profiler counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy three times, so that a counter "
                         "run can scale FETCH_SIZE / WRITE_SIZE by a kernel of known traffic")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "expert-parallel sharding (experts split over GPUs, tokens exchanged "
              "all-to-all) is not built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_moe_grouped_amd as mq
    import workloads

    dev = torch.device("cuda:0")
    mq.load()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    case = workloads.prefill_microbench(0)
    T, A, E, K, N = case.T, case.A, case.E, case.K, case.N
    flops = 2.0 * T * A * K * N
    x = to_bf16(case.x)
    idx = torch.from_numpy(case.idx).to(dev)
    wq, sc, bs = mq.mq_quantize(to_bf16(case.w), 64, 4)
    sorted_case, _ = workloads.presort(case)
    xs = to_bf16(sorted_case.x)
    idxs = torch.from_numpy(sorted_case.idx).to(dev)
    xd_np, wd_np = workloads.prefill_dense_control(0)
    xd = to_bf16(xd_np)
    wdq, sdq, bdq = mq.mq_quantize(to_bf16(wd_np), 64, 4)
    L = mq.mq_gather_qmm_workspace(T, A, 1, K, N, E, 64, 4)
    ws = torch.empty(L.total, dtype=torch.uint8, device=dev)
    out = torch.empty((T, A, 1, N), dtype=torch.bfloat16, device=dev)
    outs = torch.empty((T * A, 1, 1, N), dtype=torch.bfloat16, device=dev)
    outd = torch.empty((T * A, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn, steps, warmup):
        # the engine clock first (>= 0.3 s of back-to-back calls), then the W
        # warm-up calls; then wall clock over `steps` back-to-back calls
        # (synchronised on both sides, nothing recorded in between), then a
        # second pass with HIP events around each call on the launch stream
        # for the per-call time
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            for _ in range(50):
                fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ev_ms = [a.elapsed_time(b) for a, b in ev]
        return wall, float(np.mean(ev_ms)), float(np.median(ev_ms))

    gather = lambda: mq.mq_gather_qmm(x, wq, sc, bs, idx, True, 64, 4, False, out=out, workspace=ws)
    gather_sorted = lambda: mq.mq_gather_qmm(xs, wq, sc, bs, idxs, True, 64, 4, True, out=outs,
                                             workspace=ws)
    wsd = torch.empty(mq.mq_qmm_workspace(T * A, K, 64), dtype=torch.uint8, device=dev)
    dense = lambda: mq.mq_qmm(xd, wdq, sdq, bdq, True, 64, 4, out=outd, workspace=wsd)
    gemm_only = lambda: mq.mq_gather_qmm_routed(x, wq, sc, bs, A, ws, True, 64, 4, out=out)

    # the timed call's output, checked against the oracle on a sample before
    # anything is timed (the cpu_baseline leg)
    gather()
    torch.cuda.synchronize()
    cpu, parity, cpu_c = None, None, None
    if not args.no_cpu_baseline:
        got = (out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16)
        got = got.view(np.float32).astype(np.float64).reshape(-1, N)
        _progress("parity check and CPU oracle timing")
        cpu, parity = cpu_baseline(case, got, args.cpu_sample_tokens, args.cpu_seconds)
        _progress("fp32 C oracle timing")
        cpu_c = c_oracle_baseline(case, got, args.cpu_sample_tokens, args.cpu_seconds)
        if not parity["pass"]:
            print(f"bench.py: the timed call's output fails the parity gate: {parity}",
                  file=sys.stderr)
            sys.exit(1)

    # rotated order across variants (as in the sm_86 comment on the page), headline last
    _progress("prefill shape: sorted, dense control, GEMM alone, headline")
    _, sorted_ev, _ = timed(gather_sorted, args.steps, args.warmup)
    _, dense_ev, _ = timed(dense, args.steps, args.warmup)
    mq.mq_gather_route(idx, E, 1, workspace=ws)
    mq.mq_gather_sums(x, A, E, ws)
    _, gemm_ev, gemm_med = timed(gemm_only, args.steps, args.warmup)
    wall, call_ev, call_med = timed(gather, args.steps, args.warmup)

    ms_per_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12
    gemm_tflops = flops / (gemm_ev * 1e-3) / 1e12
    dense_tflops = flops / (dense_ev * 1e-3) / 1e12
    # algorithmic bytes of one GEMM launch: codes + scales + biases of the touched
    # experts, x rows once, output rows once
    touched = int(np.unique(case.idx).size)
    alg_bytes = touched * N * (K // 2 + 2 * 2 * K // 64) + T * A * K * 2 + T * A * N * 2

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill microbench: T=2048 A=8 E=64 K=2048 N=768, x ~ N(0,1) bf16, "
                               "W ~ N(0,1) affine 4-bit gs64, uniform routing, unsorted indices",
                   "T": T, "A": A, "E": E, "K": K, "N": N, "bits": 4, "group_size": 64},
        "mfma_peak_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("gather_gemm_prefill_T2048_A8_E64_K2048_N768.md"),
                     "kernel": "gather_gemm_kernel<128,4,64,4>",
                     "kernel_ms": round(gemm_ev, 4), "kernel_ms_median": round(gemm_med, 4),
                     "algorithmic_flops": flops, "algorithmic_bytes": alg_bytes,
                     "hbm_frac_at_kernel_time": round(alg_bytes / (gemm_ev * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "call_ms_events": round(call_ev, 4),
        # HBM bytes of one whole call (route_count + route_scatter with the row
        # sums of x + GEMM), from the same counter runs
        "call_traffic": recorded_traffic(
            "gather_gemm_prefill_T2048_A8_E64_K2048_N768.md", "call_traffic_bytes",
            ("quantized_moe_grouped_amd/csrc/gemm.hip", "quantized_moe_grouped_amd/csrc/route.hip")),
        "route_ms_est": round(call_ev - gemm_ev, 4),
        "sorted": {"value": round(flops / (sorted_ev * 1e-3) / 1e12, 2), "ms": round(sorted_ev, 4)},
        "dense_control": {"value": round(dense_tflops, 2), "ms": round(dense_ev, 4),
                          "shape": "x [16384, 2048] x quantised [768, 2048], 4-bit gs64"},
        "gather_vs_dense": round(value / dense_tflops, 4),
    }
    _progress("calibration probes")
    peaks = measured_peaks(mq, torch, dev)
    res["measured_peaks"] = peaks
    res["roofline"]["frac_of_measured_peak"] = round(gemm_tflops / peaks["mfma_bf16_TFLOPs"], 4)
    if not args.no_small_m:
        _progress("small-M decode shapes")
        res["small_m"] = small_m_bench(mq, torch, np, workloads, dev, max(10, min(args.steps, 100)),
                                       graphs=not args.no_graphs)
    if not args.no_sweeps:
        _progress("short_run_sweep")
        res["short_run_sweep"] = short_run_sweep_bench(mq, torch, np, workloads, dev, 20)
        _progress("mixtral_ffn")
        res["mixtral_ffn"] = mixtral_bench(mq, torch, np, workloads, dev, 10)
        _progress("gather_qmm_transpose0")
        res["gather_qmm_transpose0"] = gather_nn_bench(mq, torch, np, workloads, dev, 50)
        _progress("gather_mm_bf16")
        res["gather_mm_bf16"] = gather_mm_bench(mq, torch, np, workloads, dev, 50)
        _progress("gather_qmm_mxfp4")
        res["gather_qmm_mxfp4"] = gather_mx_bench(mq, torch, np, workloads, dev, 50)
        _progress("gather_qmm_mxfp8")
        res["gather_qmm_mxfp8"] = gather_mx_bench(mq, torch, np, workloads, dev, 50, bits=8)
        _progress("gather_qmm_nvfp4")
        res["gather_qmm_nvfp4"] = gather_nv_bench(mq, torch, np, workloads, dev, 50)
        _progress("mixtral_gate_up_glu")
        res["mixtral_gate_up_glu"] = glu_bench(mq, torch, np, workloads, dev, 10)
    if cpu is not None:
        # the reported baseline: the fp32 C oracle (the plain loop-nest form),
        # with the fp64 numpy oracle (the parity reference) beside it
        res["cpu_baseline"] = dict(cpu_c, numpy_fp64=cpu)
        res["parity"] = parity
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
