"""GPU-vs-oracle parity of the deployment calls through the C ABI (needs an
MI355X): the prefill -> decode handoff (final state), one decode token
(readout, update, and the fused update-then-readout step), and a prefill by
the scan followed by decode steps, which must reproduce the whole-sequence
scan.

Tolerances (relative-max error, as in parity_util):
  y          TOL of the io dtype (fp64 1e-10, fp32 1e-4, bf16 2e-2)
  state      fp64 1e-10; fp32 state (fp32 and bf16 io) 1e-4 -- the inputs are
             exact in the io dtype, so the only error is fp32 rounding of the
             accumulation; at T = 4096 tokens 1e-3 (T * 2^-24 = 2.4e-4, x4).
             The matrix-core hand-over (bf16, d_in = d_out in {64, 128}) takes
             the decay-scaled g as a pair of bf16 MFMA operands (value and
             remainder, about 2^-17 per term) against the exact bf16 x: the
             same bounds as the fp32 route.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_scans_amd as ws
from parity_util import TOL, TORCH_IO, host, relmax, to_device
from weight_scans_amd.synth import CONFIGS, Workload, make_inputs, round_to

pytestmark = pytest.mark.gpu

STATE_TOL = {"f64": 1e-10, "f32": 1e-4, "bf16": 1e-4}


def hand_over_tol(io, d_in, d_out, flags=0):
    # the matrix-core route (bf16, d_in = d_out in {64, 128}) and the vector
    # route are held to the same bound
    return STATE_TOL[io]


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    ws.lib()


def inputs(io, B, H, T, d_in, d_out, seed, alpha="base"):
    w = Workload("dec", B, H, T, d_in, d_out, io, alpha, "gauss", seed)
    inp = make_inputs(w)
    return inp, to_device(inp, io)


def state_dtype(io):
    return ws.gate_dtype(TORCH_IO[io])


@pytest.mark.parametrize("io,B,H,T,d_in,d_out,flags", [
    ("f64", 2, 3, 150, 32, 32, 0),
    ("f32", 2, 2, 200, 64, 64, 0),
    ("bf16", 2, 3, 300, 128, 128, 0),             # matrix cores
    ("bf16", 2, 3, 300, 128, 128, ws.GL_FLAG_GENERIC),
    ("bf16", 1, 2, 130, 64, 64, 0),
    ("bf16", 1, 2, 77, 37, 19, 0),      # ragged sizes, a partial last chunk
    ("f32", 1, 1, 5, 1, 128, 0),        # d_in = 1
    ("f64", 1, 2, 70, 80, 40, 0),       # 6 rows per thread, scalar LDS reads
    ("f32", 2, 1, 45, 100, 24, 0),      # 8 rows per thread, idle threads
    ("f64", 1, 2, 0, 8, 8, 0),          # no tokens: the zero adaptation
    ("bf16", 1, 2, 0, 64, 64, 0),
])
def test_final_state_parity(io, B, H, T, d_in, d_out, flags):
    say(f"final_state io={io} B={B} H={H} T={T} d_in={d_in} d_out={d_out} flags={flags}")
    inp, dev = inputs(io, B, H, T, d_in, d_out, seed=500 + T)
    S = ws.gl_scan_final_state(dev["x"], dev["g"], dev["eta"], dev["alpha"], flags=flags)
    torch.cuda.synchronize()
    want = oracle.final_state(inp["x"], inp["g"], inp["eta"], inp["alpha"])
    if T == 0:
        assert torch.count_nonzero(S).item() == 0
    else:
        err = relmax(host(S), want)
        assert err <= hand_over_tol(io, d_in, d_out, flags), err


def decode_case(io, B, H, d_in, d_out, seed):
    """One token's inputs and a cached adaptation from a 20-token prefix, as
    exact values of the device types (numpy fp64) and device tensors."""
    inp, dev = inputs(io, B, H, 21, d_in, d_out, seed)
    S = oracle.final_state(*(inp[k][:, :, :20] for k in ("x", "g", "eta", "alpha")))
    S = round_to(S, "f64" if io == "f64" else "f32")
    host_in = {k: inp[k][:, :, 20] for k in ("x", "g", "eta", "alpha")}
    host_in["W0"], host_in["S"] = inp["W0"], S
    dev_in = {k: dev[k][:, :, 20].contiguous() for k in ("x", "g", "eta", "alpha")}
    dev_in["W0"] = dev["W0"]
    dev_in["S"] = torch.from_numpy(S).to(device="cuda", dtype=state_dtype(io)).contiguous()
    return host_in, dev_in


@pytest.mark.parametrize("io,B,H,d_in,d_out", [
    ("f64", 2, 3, 64, 64),
    ("f32", 3, 2, 128, 128),
    ("bf16", 2, 4, 128, 128),
    ("bf16", 4, 16, 128, 128),      # the 1.3B-model shape
    ("bf16", 1, 3, 37, 100),        # ragged
    ("f32", 2, 1, 1, 3),
    ("f64", 2, 2, 12, 20),          # rows of 3 four-element groups (no butterfly readout)
    ("bf16", 1, 2, 4, 128),         # one group per row
    ("f32", 1, 2, 8, 7),
])
def test_decode_step_parity(io, B, H, d_in, d_out):
    say(f"decode step io={io} B={B} H={H} d_in={d_in} d_out={d_out}")
    h, d = decode_case(io, B, H, d_in, d_out, seed=600 + d_in)
    y = ws.gl_decode_readout(d["x"], d["W0"], d["S"])
    ws.gl_decode_update(d["x"], d["g"], d["eta"], d["alpha"], d["S"])
    torch.cuda.synchronize()
    y_want = oracle.decode_readout(h["x"], h["W0"], h["S"])
    S_want = oracle.decode_update(h["x"], h["g"], h["eta"], h["alpha"], h["S"])
    ey, es = relmax(host(y), y_want), relmax(host(d["S"]), S_want)
    assert ey <= TOL[io], ey
    assert es <= STATE_TOL[io], es


@pytest.mark.parametrize("io,B,H,d_in,d_out", [
    ("bf16", 4, 16, 128, 128),      # fused, one pass over the state
    ("f64", 2, 3, 64, 64),
    ("f32", 1, 2, 4, 9),
    ("bf16", 1, 3, 37, 100),        # no vector layout: update, then readout
    ("f32", 2, 2, 12, 20),
])
def test_fused_step_parity(io, B, H, d_in, d_out):
    say(f"fused step io={io} B={B} H={H} d_in={d_in} d_out={d_out}")
    h, d = decode_case(io, B, H, d_in, d_out, seed=800 + d_in)
    # the next token: another draw of the same distributions
    _, nxt = inputs(io, B, H, 1, d_in, d_out, seed=900 + d_in)
    x_next = nxt["x"][:, :, 0].contiguous()
    y = ws.gl_decode_step(d["x"], d["g"], d["eta"], d["alpha"], x_next, d["W0"], d["S"])
    torch.cuda.synchronize()
    S_want = oracle.decode_update(h["x"], h["g"], h["eta"], h["alpha"], h["S"])
    y_want = oracle.decode_readout(host(x_next), h["W0"], S_want)
    ey, es = relmax(host(y), y_want), relmax(host(d["S"]), S_want)
    assert ey <= TOL[io], ey
    assert es <= STATE_TOL[io], es


@pytest.mark.parametrize("io,d,fused", [("f64", 32, False), ("f32", 64, False),
                                        ("bf16", 64, False), ("bf16", 128, False),
                                        ("f32", 64, True), ("bf16", 128, True)])
def test_prefill_then_decode_matches_the_whole_scan(io, d, fused):
    # the scan over the first T0 tokens, the handoff, then one token at a time
    # (fused: the first token's readout, then update-and-readout steps, and
    # the last token's update)
    B, H, T, T0 = 2, 3, 300, 237
    say(f"prefill+decode io={io} d={d} T0={T0} T={T} fused={fused}")
    inp, dev = inputs(io, B, H, T, d, d, seed=700 + d)
    pre = {k: dev[k][:, :, :T0].contiguous() for k in ("x", "g", "eta", "alpha")}
    y_pre, _ = ws.gl_scan_fwd(pre["x"], pre["g"], pre["eta"], pre["alpha"], dev["W0"],
                              save=False)
    S = ws.gl_scan_final_state(pre["x"], pre["g"], pre["eta"], pre["alpha"])
    ys = [y_pre]
    tok = lambda k, t: dev[k][:, :, t].contiguous()  # noqa: E731
    for t in range(T0, T):
        if not fused:
            ys.append(ws.gl_decode_readout(tok("x", t), dev["W0"], S)[:, :, None])
            ws.gl_decode_update(tok("x", t), tok("g", t), tok("eta", t), tok("alpha", t), S)
        elif t == T0:
            ys.append(ws.gl_decode_readout(tok("x", t), dev["W0"], S)[:, :, None])
        else:
            ys.append(ws.gl_decode_step(tok("x", t - 1), tok("g", t - 1), tok("eta", t - 1),
                                        tok("alpha", t - 1), tok("x", t), dev["W0"],
                                        S)[:, :, None])
    if fused:
        ws.gl_decode_update(tok("x", T - 1), tok("g", T - 1), tok("eta", T - 1),
                            tok("alpha", T - 1), S)
    y = torch.cat(ys, dim=2)
    torch.cuda.synchronize()
    y_want = oracle.fwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], nthreads=8)
    S_want = oracle.final_state(inp["x"], inp["g"], inp["eta"], inp["alpha"])
    ey, es = relmax(host(y), y_want), relmax(host(S), S_want)
    assert ey <= TOL[io], ey
    assert es <= hand_over_tol(io, d, d), es


def test_final_state_full_size_sampled():
    # the 1.3B-model workload (B=4, H=16, T=4096, d=128, bf16), every head on
    # the GPU, three heads against the oracle
    w = CONFIGS["c4"]
    say(f"final_state full size {w}")
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    S = host(ws.gl_scan_final_state(dev["x"], dev["g"], dev["eta"], dev["alpha"]))
    Sg = host(ws.gl_scan_final_state(dev["x"], dev["g"], dev["eta"], dev["alpha"],
                                     flags=ws.GL_FLAG_GENERIC))
    for b, h in ((0, 0), (1, 7), (3, 15)):
        _, want = oracle.seq_fwd(inp["x"][b, h], inp["g"][b, h], inp["eta"][b, h],
                                 inp["alpha"][b, h], np.zeros((w.d_out, w.d_in)))
        err, errg = relmax(S[b, h], want), relmax(Sg[b, h], want)
        assert err <= 1e-3 and errg <= 1e-3, (b, h, err, errg)


def test_empty_batch_is_a_noop():
    x = torch.empty((0, 2, 8), dtype=torch.float32, device="cuda")
    S = torch.empty((0, 2, 4, 8), dtype=torch.float32, device="cuda")
    W0 = torch.zeros((2, 4, 8), dtype=torch.float32, device="cuda")
    assert ws.gl_decode_readout(x, W0, S).shape == (0, 2, 4)


def test_decode_steps_replay_in_a_hip_graph():
    # a serving loop captured once and replayed: eight fused steps on fixed
    # buffers; every replay (with eager work in between) matches the eager
    # run bit for bit (the decode kernels clear nothing with memset nodes)
    io, B, H, d, K = "bf16", 2, 4, 128, 8
    say(f"decode graph io={io} B={B} H={H} d={d} K={K}")
    _, dev = inputs(io, B, H, K + 1, d, d, seed=1900)
    S0 = ws.gl_scan_final_state(dev["x"], dev["g"], dev["eta"], dev["alpha"])
    tok = lambda k, i: dev[k][:, :, i].contiguous()  # noqa: E731
    toks = [{k: tok(k, i) for k in ("x", "g", "eta", "alpha")} for i in range(K + 1)]
    ys_e = [torch.empty((B, H, d), dtype=TORCH_IO[io], device="cuda") for _ in range(K)]
    S_e = S0.clone()
    for i in range(K):
        p, n = toks[i], toks[i + 1]
        ws.gl_decode_step(p["x"], p["g"], p["eta"], p["alpha"], n["x"], dev["W0"], S_e, y=ys_e[i])
    torch.cuda.synchronize()
    ys_g = [torch.empty_like(y) for y in ys_e]
    S_g = S0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(K):
            p, n = toks[i], toks[i + 1]
            ws.gl_decode_step(p["x"], p["g"], p["eta"], p["alpha"], n["x"], dev["W0"], S_g,
                              y=ys_g[i])
    for rep in range(3):
        S_g.copy_(S0)
        for y in ys_g:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(S_g, S_e), rep
        assert all(torch.equal(a, b) for a, b in zip(ys_g, ys_e)), rep
