#!/usr/bin/env python3
"""Throughput of the GradLev fast-weight scan (forward + reverse) on one GPU.

One step = gl_scan_fwd + gl_scan_bwd over one batch of synthetic inputs of the
named workload (default: the 340M-shape layer, [B,H,T,d] = [8,16,4096,64],
bf16 io with fp32 state).  Inputs are resident in HBM before timing starts.
Before every timed step a 1 GiB buffer is read (untimed by the events) so
that neither L2 nor the 256 MB last-level cache holds the step's inputs.

Prints ONE JSON line.  `value` = tokens/s = B*T*K / sum of event-timed
(fwd + bwd) durations (tokens, not token-heads).  `roofline` reports the
dominant pass against its binding roofline using ALGORITHMIC bytes / flops
(each input read once, each output written once).  `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload on this host.

With --decode it prints instead the deployment line: one step = one new token
of every sequence of the batch, in the steady state of serving (gl_decode_step
over all sequence-heads: the previous token's update fused with the new
token's readout), starting from the hand-over state of the named workload's
prefill (gl_scan_final_state, timed once).  The separate readout and update
calls are timed too and reported beside it.  The cached adaptation stays on the
GPU between tokens, as in serving, so no flush runs between decode steps.

With --costate it prints the line of one Picard sweep of costate
reconstruction under the quadratic token loss: gl_scan_fwd driven by the
proposed costates, then gl_costate_quadratic (g~ = y - r and the per-token
consistency residuals), on the named workload, caches flushed between sweeps
as for the main line.

With --qkv it prints the line of the transpose read z_t = (W0 + D_t)^T u_t
(gl_scan_qkv_fwd with q = u, k = g, v = x, W0 transposed) on the named
workload, caches flushed between steps; its roofline is the vector ALU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12                       # B/s, MI355X HBM3E
PEAK_MATRIX = {"bf16": 2.5e15, "f32": 157.3e12, "f64": 78.6e12}  # dense flop/s
C0 = 64                                 # chunk length used to count flops



def timing_events(steps, per_step, stream):
    """HIP events for a timed loop, created before it: torch creates an
    event's HIP handle on its first record(), and a creation that stalls the
    host between two records (the runtime growing its event pool) would be
    timed as GPU work.  Recording each once here forces the creation."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(per_step)] for _ in range(steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    return ev

def algorithmic(w):
    """Bytes and flops per pass: every input read once, every output written
    once; flops of the chunked method at chunk C0."""
    e = {"bf16": 2, "f32": 4, "f64": 8}[w.dtype]
    eg = 8 if w.dtype == "f64" else 4
    n = w.B * w.H * w.T
    di, do = w.d_in, w.d_out
    dd = di * do
    dm = 0.5 * (di + do)
    fwd_b = n * (e * (di + 2 * do) + 2 * eg) + w.H * dd * e
    bwd_b = n * (e * (2 * di + 3 * do) + 4 * eg) + w.H * dd * (e + eg)
    fwd_f = n * (6 * dd + 2 * C0 * dm)
    bwd_f = n * (16 * dd + 8 * C0 * dm)
    return {"fwd": (fwd_b, fwd_f), "bwd": (bwd_b, bwd_f)}


def binding(w, nbytes, nflops):
    t_hbm = nbytes / PEAK_HBM
    t_mx = nflops / PEAK_MATRIX[w.dtype]
    if t_hbm >= t_mx:
        return "hbm", nbytes / 1e9, PEAK_HBM / 1e9, "GB/s"
    return "mfma", nflops / 1e12, PEAK_MATRIX[w.dtype] / 1e12, "TFLOP/s"


def pass_kernels(w, which, segmented, generic):
    """The kernels one pass launches (the event-timed region of that pass)."""
    if generic:
        return {"fwd": "fwd_generic", "bwd": "bwd_generic + finalize_kernel"}[which]
    if w.dtype in ("f32", "f64"):  # the fp32 / fp64 matrix-core kernels, chunk-parallel
        return {"fwd": "fwd_inc + mf_carry + fwd_chunk",
                "bwd": "bwd_inc + mf_carry + bwd_chunk + finalize_kernel"}[which]
    if which == "fwd":
        return ("fwd_mfma (state-only) + seg_combine + fwd_mfma" if segmented else "fwd_mfma")
    # the fused backward takes its own segment count: enough (segment,
    # sequence-head) work-groups for 256 CUs, at least 16 chunks each
    bh, nch = w.B * w.H, -(-w.T // 64)
    nseg = max(1, min(-(-256 // bh), nch // 16)) if bh < 256 else 1
    pre = ("bwd_lam + seg_combine + " if nseg > 4 else "bwd_lam + ") if nseg > 1 else ""
    return pre + ("bwd_f64" if w.d_in == 64 else "bwd_f128") + " + finalize_kernel"


def host_cores():
    """(threads to use, description): every CPU this process may run on
    (sched_getaffinity), and the host's CPU model."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return max(1, n), model


def cpu_baseline(w, budget_s=20.0):
    """Time the fp64 oracle (fwd + bwd) on whole sequence-heads of the same
    workload, as many as fit ~budget_s of CPU work, on every core of the
    process's affinity set."""
    import numpy as np

    import oracle
    from weight_scans_amd.synth import make_inputs

    cores, model = host_cores()
    est = 9e-9 * w.T * w.d_in * w.d_out          # s of CPU per sequence-head
    nseq = int(max(1, min(w.B * w.H, math.ceil(budget_s / max(est, 1e-9)))))
    inp = make_inputs(w)
    flat = {k: inp[k].reshape((w.B * w.H,) + inp[k].shape[2:]) for k in
            ("x", "g", "eta", "alpha", "dy")}
    heads = np.arange(nseq) % w.H
    sl = {k: np.ascontiguousarray(flat[k][:nseq][:, None]) for k in flat}
    # one sequence per "batch" entry, each with its own head's W0
    W0 = np.ascontiguousarray(inp["W0"][heads])
    t0 = time.perf_counter()
    # run as B=nseq, H=1 per head group: group the sample by head
    for h in sorted(set(heads.tolist())):
        idx = np.nonzero(heads == h)[0]
        sub = {k: np.ascontiguousarray(sl[k][idx]) for k in sl}
        oracle.fwd(sub["x"], sub["g"], sub["eta"], sub["alpha"], W0[idx[0]][None], nthreads=cores)
        oracle.bwd(sub["x"], sub["g"], sub["eta"], sub["alpha"], W0[idx[0]][None], sub["dy"],
                   nthreads=cores)
    dt = time.perf_counter() - t0
    tokens = nseq * w.T / w.H                    # token = all H heads of one position
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "affinity_cpus": cores,
            "sample": f"{nseq} of {w.B * w.H} sequence-heads (T={w.T}, d={w.d_in}), fwd+bwd, "
                      f"fp64 serial oracle, {dt:.1f} s wall on {cores} threads ({model}); "
                      f"tokens counted as sequence-heads*T/H"}


def decode_bytes(w):
    """Algorithmic bytes of one decode token over all sequence-heads:
    (readout, update, fused step).  The readout reads the state, W0 and x and
    writes y; the update reads and writes the state and reads x, g, eta and
    alpha; the fused step reads and writes the state once and reads W0, both
    tokens' x, g, eta and alpha, and writes y."""
    e = {"bf16": 2, "f32": 4, "f64": 8}[w.dtype]
    es = 8 if w.dtype == "f64" else 4
    bh, dd = w.B * w.H, w.d_in * w.d_out
    rd = bh * (dd * es + e * (w.d_in + w.d_out)) + w.H * dd * e
    up = bh * (2 * dd * es + e * (w.d_in + w.d_out) + 2 * es)
    st = bh * (2 * dd * es + e * (2 * w.d_in + 2 * w.d_out) + 2 * es) + w.H * dd * e
    return rd, up, st


def cpu_decode(w, inp, budget_s=10.0):
    """The oracle's readout + update over every sequence-head, token after
    token, for about budget_s seconds (one thread: the oracle is serial)."""
    import numpy as np

    import oracle

    S = np.zeros((w.B, w.H, w.d_out, w.d_in))
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        k = n % inp["x"].shape[0]
        oracle.decode_readout(inp["x"][k], inp["W0"], S)
        S = oracle.decode_update(inp["x"][k], inp["g"][k], inp["eta"][k], inp["alpha"][k], S)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n * w.B / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} decode tokens of all {w.B * w.H} sequence-heads "
                      f"(d={w.d_in}), fp64 serial oracle, {dt:.1f} s wall"}


def decode_main(args, w):
    import numpy as np
    import torch

    import weight_scans_amd as ws
    from weight_scans_amd.synth import make_inputs, round_to

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tio = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    gd = ws.gate_dtype(tio)
    inp = make_inputs(w)
    pre = {k: torch.from_numpy(inp[k]).to(dev, tio) for k in ("x", "g", "W0")}
    pre.update({k: torch.from_numpy(inp[k]).to(dev, gd) for k in ("eta", "alpha")})
    del inp
    # the decode tokens: one per sequence and step, all resident before timing
    K = args.warmup + args.steps + 1
    rng = np.random.Generator(np.random.PCG64(4242))
    dec = {
        "x": round_to(rng.standard_normal((K, w.B, w.H, w.d_in)) / np.sqrt(w.d_in), w.dtype),
        "g": round_to(rng.standard_normal((K, w.B, w.H, w.d_out)) / np.sqrt(w.d_out), w.dtype),
        "eta": round_to(0.1 / (1 + np.exp(-rng.normal(-1.0, 1.0, (K, w.B, w.H)))),
                        "f64" if w.dtype == "f64" else "f32"),
        "alpha": round_to(1 / (1 + np.exp(-rng.normal(3.0, 1.0, (K, w.B, w.H)))),
                          "f64" if w.dtype == "f64" else "f32"),
    }
    dd = {k: torch.from_numpy(dec[k]).to(dev, tio if k in ("x", "g") else gd) for k in dec}
    L = ws.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())  # noqa: E731
    io = {"f64": 0, "f32": 1, "bf16": 2}[w.dtype]
    state = torch.empty((w.B, w.H, w.d_out, w.d_in), dtype=gd, device=dev)
    y = torch.empty((w.B, w.H, w.d_out), dtype=tio, device=dev)
    pdesc = ws.make_desc(w.B, w.H, w.T, w.d_in, w.d_out, io)
    ddesc = ws.make_desc(w.B, w.H, 1, w.d_in, w.d_out, io)

    # the hand-over from the prefill
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(2):
        e0.record(stream)
        ws._check(L.gl_scan_final_state(ctypes.byref(pdesc), P(pre["x"]), P(pre["g"]),
                                        P(pre["eta"]), P(pre["alpha"]), P(state), sp))
        e1.record(stream)
    torch.cuda.synchronize()
    final_ms = e0.elapsed_time(e1)

    hand_over = state.clone()

    # every token's call arguments are marshalled before timing starts, so
    # the timed loop is one C call per launch (Python's argument handling
    # would otherwise take longer than a decode kernel runs)
    dp = ctypes.byref(ddesc)
    a_rd = [(dp, P(dd["x"][k]), P(pre["W0"]), P(state), P(y), sp) for k in range(K)]
    a_up = [(dp, P(dd["x"][k]), P(dd["g"][k]), P(dd["eta"][k]), P(dd["alpha"][k]), P(state), sp)
            for k in range(K)]
    a_st = [None] + [(dp, P(dd["x"][k - 1]), P(dd["g"][k - 1]), P(dd["eta"][k - 1]),
                      P(dd["alpha"][k - 1]), P(dd["x"][k]), P(pre["W0"]), P(state), P(y), sp)
                     for k in range(1, K)]
    f_rd, f_up, f_st = L.gl_decode_readout, L.gl_decode_update, L.gl_decode_step
    bad = []

    def readout(k):
        if f_rd(*a_rd[k]):
            bad.append("readout")

    def update(k):
        if f_up(*a_up[k]):
            bad.append("update")

    # tokens are issued back to back, as a serving loop does; one pair of
    # events brackets the timed tokens (events between kernels would add gaps)
    e0, e1 = timing_events(1, 2, stream)[0]

    def timed(body):
        for k in range(1, args.warmup + 1):
            body(k)
        e0.record(stream)
        for k in range(args.warmup + 1, K):
            body(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # the separate calls: readout then update of every token, and each alone
    mp = timed(lambda k: (readout(k), update(k)))
    mr = timed(readout)
    mu = timed(update)

    # the serving loop: token 0's readout, then token k-1's update fused with
    # token k's readout
    def fused_step(k):
        if f_st(*a_st[k]):
            bad.append("step")

    state.copy_(hand_over)
    readout(0)
    ms = timed(fused_step)
    tot_ms = ms * args.steps
    # the same fused steps captured once in a HIP graph and replayed (a serving
    # loop's launch path; reported beside the eager line)
    graph_ms = None
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)  # the capture stream
            for k in range(args.warmup + 1, K):
                if f_st(*(a_st[k][:-1] + (cs,))):
                    bad.append("step (captured)")
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
    except RuntimeError as exc:  # capture not available: report the eager line only
        print(f"graph replay skipped: {exc}", file=sys.stderr)
    if bad:
        raise RuntimeError(f"decode {bad[0]} call failed: {L.gl_last_error().decode()}")
    nbytes = decode_bytes(w)[2]
    achieved = nbytes / 1e9 / (ms / 1e3)
    fused = w.d_in % 4 == 0 and ((w.d_in // 4) & (w.d_in // 4 - 1)) == 0
    rec = {
        "metric": "decode tokens/s (readout + update, every sequence of the batch)",
        "value": w.B * args.steps / (tot_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": tot_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 io / fp32 state", "f32": "f32", "f64": "f64"}[w.dtype],
        "data": "synthetic (seeded; distributions of the named workload)",
        "config": {"workload": f"{w.name} decode: B={w.B} sequences, H={w.H}, "
                               f"d={w.d_in}, state handed over after T={w.T}",
                   "B": w.B, "H": w.H, "d_in": w.d_in, "d_out": w.d_out, "io": w.dtype,
                   "parallelism": "single GPU"},
        "passes_ms": {"step_mean": ms, "step_mean_graph_replay": graph_ms,
                      "separate_readout_plus_update": mp,
                      "readout_alone": mr, "update_alone": mu, "final_state_ms": final_ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": achieved / (PEAK_HBM / 1e9), "traffic": None,
                     "algorithmic_bytes": nbytes,
                     "kernel": ("decode_readout_v (fused update + readout)" if fused else
                                "decode_update + decode_readout") +
                               "; state cache-resident between tokens"},
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_decode(w, {**{k: dec[k] for k in ("x", "g", "eta", "alpha")},
                                             "W0": np.asarray(pre["W0"].double().cpu())})
    print(json.dumps(rec), flush=True)


def costate_bytes(w):
    """Algorithmic bytes of gl_costate_quadratic: y, r and g^ read once, g~
    written once, two residuals per token."""
    e = {"bf16": 2, "f32": 4, "f64": 8}[w.dtype]
    es = 8 if w.dtype == "f64" else 4
    n = w.B * w.H * w.T
    return n * (4 * e * w.d_out + 2 * es)


def cpu_costate(w, inp, R, budget_s=10.0):
    """The oracle's sweep (its serial scan, then the reconstruction) on whole
    sequence-heads for about budget_s seconds."""
    import numpy as np

    import oracle

    cores, _ = host_cores()
    G = np.zeros((1, 1, w.T, w.d_out))
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and n < w.B * w.H:
        b, h = divmod(n, w.H)
        y = oracle.fwd(inp["x"][b, h][None, None], G, inp["eta"][b, h][None, None],
                       inp["alpha"][b, h][None, None], inp["W0"][h][None], nthreads=cores)
        oracle.costate_quadratic(y, R[b, h][None, None], G)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n * w.T / w.H / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {w.B * w.H} sequence-heads (T={w.T}, d={w.d_in}), one sweep "
                      f"(fp64 scan + reconstruction), {dt:.1f} s wall; tokens counted as "
                      f"sequence-heads*T/H"}


def costate_main(args, w):
    import numpy as np
    import torch

    import weight_scans_amd as ws
    from weight_scans_amd.synth import make_inputs, round_to

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tio = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    gd = ws.gate_dtype(tio)
    inp = make_inputs(w)
    R = round_to(np.random.default_rng(w.seed + 7).standard_normal(inp["g"].shape), w.dtype)
    t = {k: torch.from_numpy(inp[k]).to(dev, tio) for k in ("x", "W0")}
    t.update({k: torch.from_numpy(inp[k]).to(dev, gd) for k in ("eta", "alpha")})
    r = torch.from_numpy(R).to(dev, tio)
    g = torch.zeros_like(r)
    g_next = torch.empty_like(r)
    y = torch.empty_like(r)
    res_sq = torch.empty((w.B, w.H, w.T), dtype=gd, device=dev)
    res_max = torch.empty_like(res_sq)
    io = {"f64": 0, "f32": 1, "bf16": 2}[w.dtype]
    desc = ws.make_desc(w.B, w.H, w.T, w.d_in, w.d_out, io)
    fws, _ = ws.workspace_size(desc, False)
    wsb = torch.empty(max(fws, 16), dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    L = ws.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())  # noqa: E731

    def sweep(ev=None):
        nonlocal g, g_next
        if ev:
            ev[0].record(stream)
        ws._check(L.gl_scan_fwd(ctypes.byref(desc), P(t["x"]), P(g), P(t["eta"]), P(t["alpha"]),
                                P(t["W0"]), P(y), None, P(wsb), fws, sp))
        if ev:
            ev[1].record(stream)
        ws._check(L.gl_costate_quadratic(ctypes.byref(desc), P(y), P(r), P(g), P(g_next),
                                         P(res_sq), P(res_max), sp))
        if ev:
            ev[2].record(stream)
        g, g_next = g_next, g

    for _ in range(args.warmup):
        sweep()
    ev = timing_events(args.steps, 3, stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        sweep(ev[i])
    torch.cuda.synchronize()
    tf = [a.elapsed_time(b) for a, b, _ in ev]
    tc = [b.elapsed_time(c) for _, b, c in ev]
    mf, mc = sum(tf) / len(tf), sum(tc) / len(tc)
    tot_ms = sum(tf) + sum(tc)
    nbytes = costate_bytes(w)
    achieved = nbytes / 1e9 / (mc / 1e3)
    rec = {
        "metric": "tokens/s per Picard sweep (forward scan + costate reconstruction)",
        "value": w.B * w.T * args.steps / (tot_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": tot_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 io / fp32 state", "f32": "f32", "f64": "f64"}[w.dtype],
        "data": "synthetic (seeded; distributions of the named workload; targets N(0,1))",
        "config": {"workload": f"{w.name}: [B,H,T,d]=[{w.B},{w.H},{w.T},{w.d_in}] "
                               f"{w.dtype}, quadratic token loss",
                   "B": w.B, "H": w.H, "T": w.T, "d_in": w.d_in, "d_out": w.d_out,
                   "io": w.dtype, "parallelism": "single GPU"},
        "passes_ms": {"fwd_mean": mf, "costate_mean": mc},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": achieved / (PEAK_HBM / 1e9), "traffic": None,
                     "algorithmic_bytes": nbytes,
                     "kernel": "costate_k (the scan's own roofline is the main bench line)"},
        "last_res_max": float(res_max.max()),
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_costate(w, inp, R)
    print(json.dumps(rec), flush=True)


# vector ALU flop/s without packed-fp32 instructions (the library is built with
# them disabled): 256 CUs x 4 SIMDs x 16 lanes x 2 (fma) x 2.4 GHz; fp64 the same
PEAK_VALU = {"bf16": 78.6e12, "f32": 78.6e12, "f64": 78.6e12}


def qkv_bwd_main(args, w):
    """The reverse scan of the transpose read: gl_scan_qkv_bwd with q = u,
    k = g, v = x, W0 read transposed, upstream dz seeded N(0, 1)."""
    import numpy as np
    import torch

    import oracle
    import weight_scans_amd as ws
    from weight_scans_amd.synth import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tio = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    gd = ws.gate_dtype(tio)
    inp = make_inputs(w)
    dz_h = np.random.default_rng(w.seed + 77).standard_normal(inp["x"].shape)
    t = {k: torch.from_numpy(inp[k]).to(dev, tio) for k in ("x", "g", "W0", "dy")}
    t.update({k: torch.from_numpy(inp[k]).to(dev, gd) for k in ("eta", "alpha")})
    t["dz"] = torch.from_numpy(dz_h).to(dev, tio)
    dq, dk, dv = torch.empty_like(t["dy"]), torch.empty_like(t["g"]), torch.empty_like(t["x"])
    deta, dalpha = torch.empty_like(t["eta"]), torch.empty_like(t["alpha"])
    dW0 = torch.empty((w.H, w.d_out, w.d_in), dtype=gd, device=dev)
    io = {"f64": 0, "f32": 1, "bf16": 2}[w.dtype]
    flags = ws.GL_FLAG_GENERIC if args.generic else 0
    desc = ws.make_desc(w.B, w.H, w.T, w.d_out, w.d_in, io, flags=flags)
    on_mfma = w.dtype == "bf16" and w.d_in == w.d_out and w.d_in in (64, 128) and not args.generic
    n = ctypes.c_size_t()
    ws._check(ws.lib().gl_scan_qkv_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    wsb = torch.empty(max(n.value, 16), dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    # the plain copy of known size that calibrates FETCH_SIZE / WRITE_SIZE
    calib_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.neg(calib_src, out=calib_dst)  # 256 MiB in, 256 MiB out
    torch.cuda.synchronize()
    del calib_src, calib_dst
    L = ws.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())  # noqa: E731

    def step():
        ws._check(L.gl_scan_qkv_bwd(ctypes.byref(desc), P(t["dy"]), P(t["g"]), P(t["x"]),
                                    P(t["eta"]), P(t["alpha"]), P(t["W0"]), 1, P(t["dz"]),
                                    P(dq), P(dk), P(dv), P(deta), P(dalpha), P(dW0), P(wsb),
                                    n.value, sp))

    for _ in range(args.warmup):
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        step()
    ev = timing_events(args.steps, 2, stream)
    for i in range(args.steps):
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in ev]
    ms = sum(ts) / len(ts)
    # dk = d_out (q = u, k = g), dv = d_in (v = x, upstream dz).  Algorithmic
    # bytes per token-head: q, k, v, dz read and dq, dk, dv written once
    # (e (4 dk + 3 dv)), eta, alpha read and deta, dalpha written (4 eg);
    # W0 read and dW0 written once per head.  Flops of the chunked method:
    # 16 dk dv + 8 64 (dk + dv) / 2 per token-head.
    e = {"bf16": 2, "f32": 4, "f64": 8}[w.dtype]
    eg = 8 if w.dtype == "f64" else 4
    nt = w.B * w.H * w.T
    nflops = nt * (16 * w.d_in * w.d_out + 8 * 64 * (w.d_in + w.d_out) // 2)
    nbytes = nt * (e * (4 * w.d_out + 3 * w.d_in) + 4 * eg) + w.H * w.d_in * w.d_out * (e + eg)
    if on_mfma:
        # chunk-parallel on the matrix cores: bound by HBM (its flops take
        # about a tenth of the HBM time at the bf16 matrix peak)
        roof = {"bound": "hbm", "achieved": nbytes / 1e9 / (ms / 1e3), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "traffic": None, "algorithmic_bytes": nbytes,
                "algorithmic_flops": nflops,
                "kernel": f"fwd_mfma<{w.d_in}> state pass + qkv_bwd_inc<{w.d_in}> + "
                          f"qkv_grp_carry + qkv_bwd_chunk<{w.d_in}> + finalize_kernel "
                          "(whole reverse pass)"}
    else:
        # the vector-ALU kernels: the binding peak is the fp32 (fp64) vector rate
        roof = {"bound": "alu", "achieved": nflops / 1e12 / (ms / 1e3),
                "peak": PEAK_VALU[w.dtype] / 1e12, "unit": "TFLOP/s", "traffic": None,
                "algorithmic_flops": nflops, "algorithmic_bytes": nbytes,
                "kernel": "fwd_generic (states) + bwd_generic + finalize_kernel (vector ALU)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = {
        "metric": "tokens/s (reverse scan of the transpose read)",
        "value": w.B * w.T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 io / fp32 state", "f32": "f32", "f64": "f64"}[w.dtype],
        "data": "synthetic (seeded; distributions of the named workload; u ~ the dy draw)",
        "config": {"workload": f"{w.name}: [B,H,T,d]=[{w.B},{w.H},{w.T},{w.d_in}] "
                               f"{w.dtype}, gradients of z_t = (W0 + D_t)^T u_t",
                   "B": w.B, "H": w.H, "T": w.T, "d_in": w.d_in, "d_out": w.d_out,
                   "io": w.dtype, "parallelism": "single GPU"},
        "roofline": roof,
        "passes_ms": {"mean": ms, "median": statistics.median(ts), "min": min(ts), "max": max(ts),
                      "each": [round(x, 5) for x in ts]},
    }
    if not args.no_cpu:
        W0T = np.ascontiguousarray(np.transpose(inp["W0"], (0, 2, 1)))
        k_, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0 and k_ < w.B * w.H:
            b, h = divmod(k_, w.H)
            sl = lambda a: a[b:b + 1, h:h + 1]  # noqa: E731
            oracle.qkv_bwd(sl(inp["dy"]), sl(inp["g"]), sl(inp["x"]), sl(inp["eta"]),
                           sl(inp["alpha"]), W0T[h:h + 1], sl(dz_h))
            k_ += 1
        wall = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": k_ * w.T / w.H / wall, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{k_} of {w.B * w.H} sequence-heads (T={w.T}), "
                                         f"fp64 numpy token loop, {wall:.1f} s wall; "
                                         f"tokens counted as sequence-heads*T/H"}
    print(json.dumps(rec), flush=True)


def qkv_main(args, w):
    import numpy as np
    import torch

    import oracle
    import weight_scans_amd as ws
    from weight_scans_amd.synth import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tio = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    gd = ws.gate_dtype(tio)
    inp = make_inputs(w)
    t = {k: torch.from_numpy(inp[k]).to(dev, tio) for k in ("x", "g", "W0", "dy")}
    t.update({k: torch.from_numpy(inp[k]).to(dev, gd) for k in ("eta", "alpha")})
    z = torch.empty_like(t["x"])
    io = {"f64": 0, "f32": 1, "bf16": 2}[w.dtype]
    # transpose read: q = u (length d_out), k = g, v = x (length d_in)
    flags = ws.GL_FLAG_GENERIC if args.generic else 0
    desc = ws.make_desc(w.B, w.H, w.T, w.d_out, w.d_in, io, flags=flags)
    on_mfma = (w.dtype == "bf16" and w.d_in == w.d_out and w.d_in in (64, 128)
               and not args.generic)
    nws = ctypes.c_size_t()
    ws._check(ws.lib().gl_scan_qkv_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(nws)))
    qws = torch.empty(max(nws.value, 16), dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    # the plain copy of known size that calibrates FETCH_SIZE / WRITE_SIZE
    calib_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.neg(calib_src, out=calib_dst)  # 256 MiB in, 256 MiB out
    torch.cuda.synchronize()
    del calib_src, calib_dst
    L = ws.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())  # noqa: E731

    def step():
        ws._check(L.gl_scan_qkv_fwd_ws(ctypes.byref(desc), P(t["dy"]), P(t["g"]), P(t["x"]),
                                       P(t["eta"]), P(t["alpha"]), P(t["W0"]), 1, P(z), P(qws),
                                       nws.value, sp))

    for _ in range(args.warmup):  # the same sequence as a timed step, flush included
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        step()
    ev = timing_events(args.steps, 2, stream)
    for i in range(args.steps):
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in ev]
    ms = sum(ts) / len(ts)
    # 4 d_in d_out flops per token and head: the readout's and the rank-one
    # update's multiply-adds
    nflops = 4 * w.B * w.H * w.T * w.d_in * w.d_out
    if on_mfma:
        # the chunked matrix-core kernel: bound by HBM; algorithmic bytes per
        # token-head u, g, x read and z written once (e (2 d_out + 2 d_in)) and
        # the two gates (fp32), plus W0 once; its flops (6 d^2 + 2 64 d per
        # token-head) take a fifth of the HBM time at the bf16 matrix peak
        e = 2
        nbytes = (w.B * w.H * w.T * (e * (2 * w.d_out + 2 * w.d_in) + 8)
                  + w.H * w.d_in * w.d_out * e)
        kern = ("fwd_mfma<64> with a read tile of its own (chunked, matrix cores)" if w.d_in == 64
                else "fwd_mfma<128> state pass (a state per group of eight chunks) + qkv_group "
                "(groups in parallel, each walked in order; matrix cores)")
        roof = {"bound": "hbm", "achieved": nbytes / 1e9 / (ms / 1e3), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "traffic": None, "algorithmic_bytes": nbytes, "kernel": kern}
    else:
        achieved = nflops / 1e12 / (ms / 1e3)
        peak = PEAK_VALU[w.dtype] / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "traffic": None, "algorithmic_flops": nflops,
                "kernel": "qkv_fwd_k (tokens in order, rows across lanes)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = {
        "metric": "tokens/s (transpose read of the adapted weight)",
        "value": w.B * w.T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 io / fp32 state", "f32": "f32", "f64": "f64"}[w.dtype],
        "data": "synthetic (seeded; distributions of the named workload; u ~ the dy draw)",
        "config": {"workload": f"{w.name}: [B,H,T,d]=[{w.B},{w.H},{w.T},{w.d_in}] "
                               f"{w.dtype}, z_t = (W0 + D_t)^T u_t",
                   "B": w.B, "H": w.H, "T": w.T, "d_in": w.d_in, "d_out": w.d_out,
                   "io": w.dtype, "parallelism": "single GPU"},
        "roofline": roof,
        "passes_ms": {"mean": ms, "median": statistics.median(ts), "min": min(ts), "max": max(ts),
                      "each": [round(x, 5) for x in ts]},
    }
    if not args.no_cpu:
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        W0T = np.ascontiguousarray(np.transpose(inp["W0"], (0, 2, 1)))
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0 and n < w.B * w.H:
            b, h = divmod(n, w.H)
            sl = lambda k: inp[k][b:b + 1, h:h + 1]  # noqa: E731
            oracle.qkv_fwd(sl("dy"), sl("g"), sl("x"), sl("eta"), sl("alpha"), W0T[h:h + 1])
            n += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": n * w.T / w.H / dt, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} of {w.B * w.H} sequence-heads (T={w.T}), fp64 "
                                         f"numpy loop, {dt:.1f} s wall; tokens counted as "
                                         f"sequence-heads*T/H"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-flush", action="store_true", help="do not flush caches between steps")
    ap.add_argument("--generic", action="store_true", help="force the portable VALU kernels")
    ap.add_argument("--qkv", action="store_true",
                    help="time the transpose read (scan with its own read vector and key)")
    ap.add_argument("--qkv-bwd", action="store_true",
                    help="time the reverse scan of the transpose read (gl_scan_qkv_bwd)")
    ap.add_argument("--costate", action="store_true",
                    help="time Picard sweeps (forward scan + costate reconstruction)")
    ap.add_argument("--decode", action="store_true",
                    help="time one-token decode steps (readout + update) instead of the scan")
    ap.add_argument("--segments", type=int, default=0,
                    help="segments per sequence (0 = the library's automatic choice)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan path here has no multi-GPU "
              "implementation (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import weight_scans_amd as ws
    from weight_scans_amd.synth import CONFIGS, make_inputs

    w = CONFIGS[args.config]
    if args.decode:
        return decode_main(args, w)
    if args.costate:
        return costate_main(args, w)
    if args.qkv:
        return qkv_main(args, w)
    if args.qkv_bwd:
        return qkv_bwd_main(args, w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tio = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    gd = ws.gate_dtype(tio)
    inp = make_inputs(w)
    t = {k: torch.from_numpy(inp[k]).to(dev, tio) for k in ("x", "g", "W0", "dy")}
    t.update({k: torch.from_numpy(inp[k]).to(dev, gd) for k in ("eta", "alpha")})
    del inp
    flags = ws.GL_FLAG_GENERIC if args.generic else 0
    desc = ws.make_desc(w.B, w.H, w.T, w.d_in, w.d_out,
                        {"f64": 0, "f32": 1, "bf16": 2}[w.dtype], w.chunk, flags, args.segments)
    path = ws.path_name(desc)
    y = torch.empty((w.B, w.H, w.T, w.d_out), dtype=tio, device=dev)
    dx, dg = torch.empty_like(t["x"]), torch.empty_like(t["g"])
    deta, dalpha = torch.empty_like(t["eta"]), torch.empty_like(t["alpha"])
    dW0 = torch.empty((w.H, w.d_out, w.d_in), dtype=gd, device=dev)
    saved = torch.empty(max(ws.saved_size(desc), 16), dtype=torch.uint8, device=dev)
    fws, bws = ws.workspace_size(desc, True)
    segmented = fws > 0  # the forward needs a workspace only for segments
    wsb = torch.empty(max(fws, bws, 16), dtype=torch.uint8, device=dev)
    # cache flush between steps: a 1 GiB read (4x the memory-side cache), so
    # the inputs come from HBM.  A read leaves only clean lines behind; a fill
    # would leave its own dirty lines, whose write-back then lands inside the
    # timed kernels (measured: a 256 MB read right after a 1 GiB fill runs at
    # about 2.4 TB/s, right after a 1 GiB read at about 5.8 TB/s).
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    # one plain copy of known size (256 MiB each way): the reference that turns
    # the FETCH_SIZE / WRITE_SIZE counters of a profiled run into bytes
    calib_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.neg(calib_src, out=calib_dst)  # a plain elementwise kernel: 256 MiB in, 256 MiB out
    torch.cuda.synchronize()
    del calib_src, calib_dst
    L = ws.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())  # noqa: E731

    def fwd():
        ws._check(L.gl_scan_fwd(ctypes.byref(desc), P(t["x"]), P(t["g"]), P(t["eta"]),
                                P(t["alpha"]), P(t["W0"]), P(y), P(saved), P(wsb), fws, sp))

    def bwd():
        ws._check(L.gl_scan_bwd(ctypes.byref(desc), P(t["x"]), P(t["g"]), P(t["eta"]),
                                P(t["alpha"]), P(t["W0"]), P(t["dy"]), P(saved), P(dx), P(dg),
                                P(deta), P(dalpha), P(dW0), P(wsb), bws, sp))

    for i in range(args.warmup):  # the same sequence as a timed step, flush included
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        fwd()
        bwd()
    torch.cuda.synchronize()

    ev = timing_events(args.steps, 3, stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush_sink = torch.sum(flush)  # noqa: F841
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tf = [a.elapsed_time(b) for a, b, _ in ev]
    tb = [b.elapsed_time(c) for _, b, c in ev]
    tot_ms = sum(tf) + sum(tb)
    ms_step = tot_ms / args.steps
    tokens = w.B * w.T
    value = tokens * args.steps / (tot_ms / 1e3)

    alg = algorithmic(w)
    mf, mb = sum(tf) / len(tf), sum(tb) / len(tb)
    med = statistics.median
    dom, dom_ms = ("bwd", mb) if mb >= mf else ("fwd", mf)
    nbytes, nflops = alg[dom]
    bound, amount, peak, unit = binding(w, nbytes, nflops)
    achieved = amount / (dom_ms / 1e3)
    # roofline of the whole step (both passes against their own bounds)
    step_floor = sum(max(alg[p][0] / PEAK_HBM, alg[p][1] / PEAK_MATRIX[w.dtype]) for p in alg)

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath) and not args.generic:
        from weight_scans_amd.profiling import kernel_source_hash
        rec_t = json.load(open(tpath)).get(w.name)
        if rec_t and rec_t.get("kernel_hash") == kernel_source_hash():
            traffic = rec_t[f"{dom}_bytes"]

    rec = {
        "metric": "tokens/s (fwd+bwd scan)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 io / fp32 state", "f32": "f32", "f64": "f64"}[w.dtype],
        "data": "synthetic (seeded; distributions of the named workload)",
        "config": {"workload": f"{w.name}: [B,H,T,d]=[{w.B},{w.H},{w.T},{w.d_in}] "
                               f"{w.dtype}", "B": w.B, "H": w.H, "T": w.T, "d_in": w.d_in,
                   "d_out": w.d_out, "io": w.dtype, "kernels": path,
                   "parallelism": "single GPU"},
        "passes_ms": {"fwd_mean": mf, "bwd_mean": mb,
                      "fwd_median": med(tf), "fwd_min": min(tf), "fwd_max": max(tf),
                      "bwd_median": med(tb), "bwd_min": min(tb), "bwd_max": max(tb),
                      "fwd_each": [round(x, 5) for x in tf], "bwd_each": [round(x, 5) for x in tb]},
        "tokens_per_s_median": tokens / ((med(tf) + med(tb)) / 1e3),
        # one step (fwd + bwd pass) end to end: the figure for latency-bound
        # workloads such as a single short sequence
        "step_latency_us_median": med([a + b for a, b in zip(tf, tb)]) * 1e3,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic,
                     "algorithmic_bytes": nbytes, "algorithmic_flops": nflops,
                     "kernel": f"{dom} pass ({path}): " + pass_kernels(w, dom, segmented, args.generic),
                     "step_frac": step_floor / (ms_step / 1e3)},
        "wall_ms_per_step_incl_flush": wall * 1e3 / args.steps,
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
