#!/usr/bin/env python3
"""Throughput of the GradLev fast-weight scan (forward + reverse) on one GPU.

One step = gl_scan_fwd + gl_scan_bwd over one batch of synthetic inputs of the
named workload (default: the 340M-shape layer, [B,H,T,d] = [8,16,4096,64],
bf16 io with fp32 state).  Inputs are resident in HBM before timing starts.
Before every timed step a 1 GiB buffer is overwritten (untimed by the events)
so that neither L2 nor the 256 MB last-level cache holds the step's inputs.

Prints ONE JSON line.  `value` = tokens/s = B*T*K / sum of event-timed
(fwd + bwd) durations (tokens, not token-heads).  `roofline` reports the
dominant pass against its binding roofline using ALGORITHMIC bytes / flops
(each input read once, each output written once).  `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12                       # B/s, MI355X HBM3E
PEAK_MATRIX = {"bf16": 2.5e15, "f32": 157.3e12, "f64": 78.6e12}  # dense flop/s
C0 = 64                                 # chunk length used to count flops


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
    if which == "fwd":
        return ("fwd_mfma (state-only) + seg_combine + fwd_mfma" if segmented else "fwd_mfma")
    # the fused backward takes its own segment count: enough (segment,
    # sequence-head) work-groups for 256 CUs, at least 16 chunks each
    bh, nch = w.B * w.H, -(-w.T // 64)
    nseg = max(1, min(-(-256 // bh), nch // 16)) if bh < 256 else 1
    pre = ("bwd_lam + seg_combine + " if nseg > 4 else "bwd_lam + ") if nseg > 1 else ""
    return pre + ("bwd_f64" if w.d_in == 64 else "bwd_f128") + " + finalize_kernel"


def cpu_baseline(w, budget_s=20.0):
    """Time the fp64 oracle (fwd + bwd) on whole sequence-heads of the same
    workload, as many as fit ~budget_s of CPU work, on this host's cores."""
    import numpy as np

    import oracle
    from weight_scans_amd.synth import make_inputs

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
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
            "sample": f"{nseq} of {w.B * w.H} sequence-heads (T={w.T}, d={w.d_in}), fwd+bwd, "
                      f"fp64 serial oracle, {dt:.1f} s wall; tokens counted as "
                      f"sequence-heads*T/H"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-flush", action="store_true", help="do not flush caches between steps")
    ap.add_argument("--generic", action="store_true", help="force the portable VALU kernels")
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

    for i in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
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
        "passes_ms": {"fwd_mean": mf, "bwd_mean": mb, "fwd_min": min(tf), "bwd_min": min(tb)},
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
