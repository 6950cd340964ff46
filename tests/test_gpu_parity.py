"""GPU-vs-oracle parity through the C ABI (needs an MI355X).

Small workloads are compared element by element over every output; the large
ones (the 340M / 1.3B / long-context shapes) run in full on the GPU and are
compared over the whole workload (every sequence-head, every output, dW0 of
every head), and on sampled sequence-heads.  Tolerances are in parity_util.
"""
import json
import os

import numpy as np
import pytest
import torch

import weight_scans_amd as ws
from parity_util import (NAMES, TOL, compare_full, compare_sampled, error_stats, host,
                         oracle_all, oracle_sampled, relmax, run_gpu, stats_ok, to_device)
import oracle
from weight_scans_amd.synth import CONFIGS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def report(case, errs):
    """Append the measured errors to $PARITY_REPORT (JSON lines), if set."""
    path = os.environ.get("PARITY_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps({"case": str(case), "errs": errs}) + "\n")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    ws.lib()


def _full_case(w: Workload, **kw):
    say(f"case {w} {kw}")
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    gpu = run_gpu(dev, chunk=w.chunk if "chunk" not in kw else kw.pop("chunk"), **kw)
    ref = oracle_all(inp)
    errs, bad = compare_full(gpu, ref, TOL[w.dtype])
    say(f"  errs {errs}")
    report(w.name, errs)
    assert not bad, "\n".join(f"{k}: {v:.3e}" for k, v in errs.items())
    return gpu, ref


def test_c1_fp64_full():
    _full_case(CONFIGS["c1"])


def test_c1_fp64_recompute_path():
    _full_case(CONFIGS["c1"], use_saved=False)


def test_c2_fp32_full():
    # c2 as specified: fp32 throughout, chunk 64 (the fp32 matrix-core kernels)
    w = CONFIGS["c2"]
    assert w.chunk == 64
    d = ws.make_desc(w.B, w.H, w.T, w.d_in, w.d_out, ws.GL_DTYPE_F32, w.chunk)
    assert ws.path_name(d) == "mfma-f32"
    _full_case(w)


def test_c1_on_the_matrix_cores():
    w = CONFIGS["c1"]
    d = ws.make_desc(w.B, w.H, w.T, w.d_in, w.d_out, ws.GL_DTYPE_F64, w.chunk)
    assert ws.path_name(d) == "mfma-f64"


@pytest.mark.parametrize("io,d_in,d_out", [("f32", 64, 64), ("f32", 20, 50), ("f64", 32, 32),
                                           ("f64", 7, 30)])
def test_matrix_core_and_vector_paths_agree(io, d_in, d_out):
    """fp32 / fp64 on the matrix cores (chunk 64) and on the vector ALU
    (GL_FLAG_GENERIC): both within tolerance of the oracle."""
    w = Workload("mv", 2, 2, 300, d_in, d_out, io, "mix", "gauss", 2200 + d_in + d_out)
    inp = make_inputs(w)
    dev = to_device(inp, io)
    ref = oracle_all(inp)
    for flags in (0, ws.GL_FLAG_GENERIC):
        gpu = run_gpu(dev, flags=flags)
        errs, bad = compare_full(gpu, ref, TOL[io])
        say(f"  flags {flags} errs {errs}")
        assert not bad, (flags, errs)


@pytest.mark.parametrize("name,pairs,head", [
    ("c3", [(0, 0), (7, 15), (3, 9)], 5),
    ("c4", [(0, 0), (3, 15)], 7),
    ("c5", [(0, 0), (0, 11)], 3),
])
def test_large_sampled(name, pairs, head):
    w = CONFIGS[name]
    say(f"case {w}")
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    gpu = run_gpu(dev)
    ref = oracle_sampled(inp, pairs, dW0_head=head)
    errs = compare_sampled(gpu, ref, dW0_head=head)
    say(f"  errs {errs}")
    report(name, errs)
    bad = {k: e for k, e in errs.items() if not e <= TOL[w.dtype]}
    assert not bad, "\n".join(f"{k}: {v:.3e}" for k, v in errs.items())
    for n in NAMES:
        assert torch.isfinite(gpu[n]).all(), n


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_whole_workload(name):
    """Every sequence-head of the full-size workload against the oracle: the
    max-norm gate per output and per sequence-head, dW0 of every head, and the
    RMS / bias / slope statistics of every per-token output."""
    w = CONFIGS[name]
    say(f"case {w} whole workload")
    inp = make_inputs(w)
    gpu = run_gpu(to_device(inp, w.dtype))
    say("  gpu done; oracle forward + reverse scan on every sequence-head")
    ref = oracle_all(inp, nthreads=16)
    say("  oracle done")
    bad = {}
    for n in NAMES:
        got, r = host(gpu[n]), ref[n]
        st = {"relmax": relmax(got, r)}
        if n != "dW0":
            st.update(error_stats(got, r))
            # the worst sequence-head, each normalised by its own largest value
            d = np.abs(got - r).reshape(w.B * w.H, -1).max(axis=1)
            m = np.abs(r).reshape(w.B * w.H, -1).max(axis=1)
            st["relmax_worst_head"] = float(np.max(d / np.where(m > 0, m, 1.0)))
        say(f"  {n}: " + ", ".join(f"{k} {v:.2e}" for k, v in st.items()))
        report(f"{name} whole {n}", st)
        ok = st["relmax"] <= TOL[w.dtype] and st.get("relmax_worst_head", 0.0) <= TOL[w.dtype]
        if n != "dW0":
            ok = ok and stats_ok(st)
        if not ok:
            bad[n] = st
        del got, r
    assert not bad, bad


EDGE = [
    ("f64", 1, 1, 1, 8, 8), ("f64", 1, 2, 2, 5, 3), ("f64", 2, 1, 17, 1, 1),
    ("f64", 1, 2, 33, 128, 3), ("f32", 2, 2, 63, 32, 32), ("f32", 1, 3, 64, 48, 80),
    ("f32", 1, 1, 65, 64, 64), ("f32", 1, 2, 1000, 16, 24), ("bf16", 2, 2, 65, 64, 64),
    ("bf16", 1, 2, 1000, 128, 128), ("bf16", 1, 1, 2, 128, 128), ("bf16", 3, 1, 129, 40, 72),
    # the fp32 / fp64 matrix-core kernels with ragged widths (element-wise tile
    # loads) and one full width against a ragged one
    ("f32", 2, 2, 129, 64, 17), ("f32", 1, 3, 191, 33, 64), ("f64", 2, 2, 129, 32, 31),
    ("f64", 1, 1, 64, 1, 32),
]


@pytest.mark.parametrize("io,B,H,T,di,do", EDGE)
def test_edge_shapes(io, B, H, T, di, do):
    _full_case(Workload("edge", B, H, T, di, do, io, "mix", "gauss", 500 + T + di))


# Segmented scan (sequences cut into segments scanned by separate work-groups,
# then combined): 8 chunks with a ragged tail; 3 segments start at an odd
# chunk, 5 requested give 4 of 2 chunks, 8 give one chunk each.
SEGMENTED = [(64, 3), (64, 5), (64, 8), (128, 3), (128, 5), (128, 8)]


@pytest.mark.parametrize("d,segments", SEGMENTED)
def test_segments_full(d, segments):
    w = Workload("seg", 1, 2, 64 * 7 + 13, d, d, "bf16", "mix", "unit", 700 + d + segments)
    _full_case(w, segments=segments)


@pytest.mark.parametrize("d", [64, 128])
def test_segments_recompute_path(d):
    w = Workload("segr", 2, 1, 64 * 9 + 1, d, d, "bf16", "mix", "unit", 800 + d)
    _full_case(w, segments=4, use_saved=False)


def test_segments_and_none_agree():
    """The same inputs with and without segments: both within the bf16
    tolerance of the oracle, and close to each other."""
    w = Workload("segs", 1, 2, 64 * 16, 64, 64, "bf16", "mix", "unit", 901)
    gpu1, ref = _full_case(w, segments=1)
    gpu4, _ = _full_case(w, segments=4)
    for n in NAMES:
        assert relmax(host(gpu4[n]), host(gpu1[n])) < TOL["bf16"], n


@pytest.mark.parametrize("io", ["f64", "f32", "bf16"])
def test_identity_gates(io):
    """alpha = 1, eta = 0: y = W0 x and no adaptation gradients."""
    w = Workload("id", 2, 2, 130, 64, 64, io, "base", "gauss", 77)
    inp = make_inputs(w)
    inp["alpha"][:] = 1.0
    inp["eta"][:] = 0.0
    gpu = run_gpu(to_device(inp, io))
    ref = oracle_all(inp)
    errs, bad = compare_full(gpu, ref, TOL[io])
    assert not bad, errs
    assert float(gpu["dg"].abs().max()) == 0.0


@pytest.mark.parametrize("io,chunks", [("f64", (8, 16, 64)), ("f32", (8, 16, 32, 64)),
                                        ("bf16", (8, 16, 32))])
def test_chunk_invariance(io, chunks):
    w = Workload("ch", 1, 2, 200, 32, 32, io, "mix", "gauss", 91)
    inp = make_inputs(w)
    dev = to_device(inp, io)
    ref = oracle_all(inp)
    for c in chunks:
        gpu = run_gpu(dev, chunk=c)
        errs, bad = compare_full(gpu, ref, TOL[io])
        assert not bad, (c, errs)


@pytest.mark.parametrize("name", ["c3", "c2"])
def test_run_to_run_bitwise_determinism(name):
    w = CONFIGS[name].with_(B=2, T=1024)
    dev = to_device(make_inputs(w), w.dtype)
    a = run_gpu(dev)
    b = run_gpu(dev)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_nan_stays_in_its_sequence():
    w = Workload("nan", 3, 2, 70, 32, 32, "f32", "base", "gauss", 5)
    inp = make_inputs(w)
    dev = to_device(inp, "f32")
    clean = run_gpu(dev)
    dev["x"][1, 0, 40, 3] = float("nan")
    dirty = run_gpu(dev)
    for n in ("y", "dx", "dg", "deta", "dalpha"):
        for b in range(3):
            for h in range(2):
                if (b, h) == (1, 0):
                    continue
                assert torch.equal(clean[n][b, h], dirty[n][b, h]), (n, b, h)
    assert torch.equal(clean["dW0"][1], dirty["dW0"][1])
    assert not torch.isfinite(dirty["dW0"][0]).all()


def test_autograd_function_matches_bwd():
    w = Workload("ag", 2, 2, 90, 32, 32, "f64", "mix", "gauss", 13)
    inp = make_inputs(w)
    dev = to_device(inp, "f64")
    leaves = {k: dev[k].clone().requires_grad_(True) for k in ("x", "g", "eta", "alpha", "W0")}
    y = ws.scan(leaves["x"], leaves["g"], leaves["eta"], leaves["alpha"], leaves["W0"])
    (y * dev["dy"]).sum().backward()
    ref = oracle_all(inp)
    for k, n in (("x", "dx"), ("g", "dg"), ("eta", "deta"), ("alpha", "dalpha"), ("W0", "dW0")):
        assert relmax(host(leaves[k].grad), ref[n]) < TOL["f64"], k


@pytest.mark.parametrize("d,T", [(64, 200), (128, 130), (40, 77)])
def test_out_f32(d, T):
    """GL_FLAG_OUT_F32: bf16 inputs, y / dx / dg returned in fp32 (not rounded
    to bf16), every output within the bf16 tolerance of the oracle."""
    w = Workload("of32", 2, 2, T, d, d, "bf16", "mix", "gauss", 2100 + d)
    inp = make_inputs(w)
    dev = to_device(inp, "bf16")
    gpu = run_gpu(dev, flags=ws.GL_FLAG_OUT_F32)
    for n in ("y", "dx", "dg"):
        assert gpu[n].dtype == torch.float32, n
    ref = oracle_all(inp)
    errs, bad = compare_full(gpu, ref, TOL["bf16"])
    say(f"  errs {errs}")
    report(f"out_f32 d={d}", errs)
    assert not bad, errs
    # without the final rounding to bf16 the outputs sit closer to the oracle
    plain = run_gpu(dev)
    for n in ("y", "dx", "dg"):
        e32 = error_stats(host(gpu[n]), ref[n])["rel_rms"]
        e16 = error_stats(host(plain[n]), ref[n])["rel_rms"]
        assert e32 < e16, (n, e32, e16)


def test_empty_inputs():
    for io in ("f64", "bf16"):
        w = Workload("e", 2, 3, 0, 16, 16, io, "base", "gauss", 1)
        inp = make_inputs(w)
        dev = to_device(inp, io)
        out = run_gpu(dev)
        assert out["y"].numel() == 0
        assert out["dW0"].shape == (3, 16, 16) and float(out["dW0"].abs().max()) == 0.0
