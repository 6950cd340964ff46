"""Shared helpers for the GPU-vs-oracle parity tests.

Tolerances (relative-max error per output tensor, max|gpu - ref| / max|ref|,
computed in fp64 over the compared elements):
  fp64 io            1e-10
  fp32 io            1e-4   (no tolerance is given for fp32; this one is derived
                             from fp32 rounding over chunk-length dot products)
  bf16 io, fp32 acc  2e-2
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from weight_scans_amd import gate_dtype, gl_scan_bwd, gl_scan_fwd
from weight_scans_amd.synth import make_inputs

TOL = {"f64": 1e-10, "f32": 1e-4, "bf16": 2e-2}
TORCH_IO = {"f64": torch.float64, "f32": torch.float32, "bf16": torch.bfloat16}
NAMES = ("y", "dx", "dg", "deta", "dalpha", "dW0")


def relmax(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = float(np.max(np.abs(want))) if want.size else 0.0
    if want.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want)) / (den if den > 0 else 1.0))


# Beside the max-norm gate, bf16 results are held to statistics that a
# systematic error would move while rounding noise does not (measured: the
# relative RMS error of every output is 1e-3 .. 3e-3, bias and slope errors
# below 1e-4):
#   rel_rms = rms(gpu - ref) / rms(ref)              <= 5e-3
#   bias    = |mean(gpu - ref)| / rms(ref)             <= 1e-3
#   slope   = |<gpu, ref> / <ref, ref> - 1|            <= 2e-3
BF16_STATS = {"rel_rms": 5e-3, "bias": 1e-3, "slope": 2e-3}


def error_stats(got, want) -> dict:
    got = np.asarray(got, np.float64).ravel()
    want = np.asarray(want, np.float64).ravel()
    if want.size == 0:
        return {"rel_rms": 0.0, "bias": 0.0, "slope": 0.0}
    rms = float(np.sqrt(np.mean(want * want)))
    if rms == 0.0:
        rms = 1.0
    d = got - want
    ww = float(np.dot(want, want))
    return {"rel_rms": float(np.sqrt(np.mean(d * d))) / rms,
            "bias": abs(float(np.mean(d))) / rms,
            "slope": abs(float(np.dot(got, want)) / ww - 1.0) if ww > 0 else 0.0}


def stats_ok(stats: dict) -> bool:
    return all(stats[k] <= v for k, v in BF16_STATS.items())


def to_device(inp: dict, io: str, device="cuda"):
    tio = TORCH_IO[io]
    gd = gate_dtype(tio)
    out = {}
    for k in ("x", "g", "W0", "dy"):
        out[k] = torch.from_numpy(inp[k]).to(device=device, dtype=tio).contiguous()
    for k in ("eta", "alpha"):
        out[k] = torch.from_numpy(inp[k]).to(device=device, dtype=gd).contiguous()
    return out


def run_gpu(dev: dict, chunk=0, flags=0, use_saved=True, segments=0):
    """Forward then backward through the C ABI; returns device tensors."""
    y, saved = gl_scan_fwd(dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"],
                           chunk=chunk, flags=flags, save=use_saved, segments=segments)
    grads = gl_scan_bwd(dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"], dev["dy"],
                        saved if use_saved else None, chunk=chunk, flags=flags,
                        segments=segments)
    torch.cuda.synchronize()
    return dict(zip(NAMES, (y,) + tuple(grads)))


def host(t) -> np.ndarray:
    return t.double().cpu().numpy()


def oracle_all(inp: dict, nthreads=8):
    y = oracle.fwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], nthreads=nthreads)
    g = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], inp["dy"],
                   nthreads=nthreads)
    return dict(zip(NAMES, (y,) + tuple(g)))


def oracle_sampled(inp: dict, pairs, dW0_head=None, nthreads=8):
    """Oracle outputs for selected (b, h) sequences, plus dW0 of one head
    (summed over the whole batch)."""
    res = {}
    for (b, h) in pairs:
        sl = {k: inp[k][b:b + 1, h:h + 1] for k in ("x", "g", "eta", "alpha", "dy")}
        W0 = inp["W0"][h:h + 1]
        y = oracle.fwd(sl["x"], sl["g"], sl["eta"], sl["alpha"], W0)
        dx, dg, de, da, _ = oracle.bwd(sl["x"], sl["g"], sl["eta"], sl["alpha"], W0, sl["dy"])
        res[(b, h)] = dict(y=y[0, 0], dx=dx[0, 0], dg=dg[0, 0], deta=de[0, 0], dalpha=da[0, 0])
    if dW0_head is not None:
        h = dW0_head
        sl = {k: inp[k][:, h:h + 1] for k in ("x", "g", "eta", "alpha", "dy")}
        *_, dW = oracle.bwd(sl["x"], sl["g"], sl["eta"], sl["alpha"], inp["W0"][h:h + 1],
                            sl["dy"], nthreads=nthreads)
        res["dW0"] = dW[0]
    return res


def compare_full(gpu: dict, ref: dict, tol: float):
    errs = {n: relmax(host(gpu[n]), ref[n]) for n in NAMES}
    bad = {n: e for n, e in errs.items() if not e <= tol}
    return errs, bad


def compare_sampled(gpu: dict, ref: dict, dW0_head=None):
    errs = {}
    for key, r in ref.items():
        if key == "dW0":
            errs["dW0"] = relmax(host(gpu["dW0"][dW0_head]), r)
            continue
        b, h = key
        for n, v in r.items():
            errs[f"{n}[{b},{h}]"] = relmax(host(gpu[n][b, h]), v)
    return errs
