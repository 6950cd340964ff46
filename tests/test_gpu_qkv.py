"""GPU-vs-oracle parity of the scan with its own read vector and write key
(transpose read and separate write key) through the C ABI (needs an MI355X).
Tolerances as the scan's (parity_util.TOL): fp64 1e-10, fp32 1e-4, bf16 2e-2;
the kernel runs the recurrence token by token in the compute type.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_scans_amd as ws
from parity_util import TOL, TORCH_IO, host, relmax, to_device
from weight_scans_amd.synth import CONFIGS, Workload, make_inputs, round_to

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    ws.lib()


def case(io, B, H, T, d_in, d_out, seed):
    w = Workload("qkv", B, H, T, d_in, d_out, io, "base", "gauss", seed)
    inp = make_inputs(w)
    return inp, to_device(inp, io)


@pytest.mark.parametrize("io,B,H,T,d_in,d_out", [
    ("f64", 2, 3, 100, 32, 32),
    ("f32", 1, 2, 200, 64, 48),
    ("bf16", 2, 2, 300, 128, 128),
    ("f32", 1, 2, 77, 37, 100),       # ragged: dk = 100 > 64, dv = 37
    ("bf16", 1, 1, 5, 1, 3),
])
def test_transpose_read_parity(io, B, H, T, d_in, d_out):
    # z_t = (W0 + D_t)^T u_t: q = u [d_out], k = g, v = x, W0 read transposed
    say(f"transpose read io={io} B={B} H={H} T={T} d_in={d_in} d_out={d_out}")
    inp, dev = case(io, B, H, T, d_in, d_out, seed=1500 + d_in)
    u = inp["dy"]  # a hidden costate at the layer output
    z = ws.transpose_read(dev["dy"], dev["g"], dev["x"], dev["eta"], dev["alpha"], dev["W0"])
    torch.cuda.synchronize()
    W0T = np.ascontiguousarray(np.transpose(inp["W0"], (0, 2, 1)))
    want = oracle.qkv_fwd(u, inp["g"], inp["x"], inp["eta"], inp["alpha"], W0T)
    err = relmax(host(z), want)
    assert err <= TOL[io], err


@pytest.mark.parametrize("io,B,H,T,d", [("f64", 2, 2, 90, 16), ("f32", 2, 3, 150, 64),
                                        ("bf16", 1, 2, 200, 128)])
def test_write_key_parity(io, B, H, T, d):
    # q = x, k = a centered key, v = g
    say(f"write key io={io} B={B} H={H} T={T} d={d}")
    inp, dev = case(io, B, H, T, d, d, seed=1600 + d)
    xb = round_to(inp["x"] - inp["x"].mean(axis=2, keepdims=True), io)
    xb_d = torch.from_numpy(xb).to("cuda", TORCH_IO[io])
    y = ws.gl_scan_qkv_fwd(dev["x"], xb_d, dev["g"], dev["eta"], dev["alpha"], dev["W0"])
    torch.cuda.synchronize()
    want = oracle.qkv_fwd(inp["x"], xb, inp["g"], inp["eta"], inp["alpha"], inp["W0"])
    err = relmax(host(y), want)
    assert err <= TOL[io], err


def test_qkv_with_equal_keys_is_the_forward_scan():
    # q = k = x, v = g: the same outputs as gl_scan_fwd (both within the
    # scan's tolerance of the oracle; here directly against each other)
    inp, dev = case("f32", 2, 2, 130, 64, 64, seed=1700)
    y1 = ws.gl_scan_qkv_fwd(dev["x"], dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"])
    y2, _ = ws.gl_scan_fwd(dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"], save=False)
    torch.cuda.synchronize()
    assert relmax(host(y1), host(y2)) <= 1e-4


def test_transpose_read_full_size_sampled():
    # the 340M-model shape (B=8, H=16, T=4096, d=64, bf16), every head on the
    # GPU, two heads against the oracle
    w = CONFIGS["c3"]
    say(f"transpose read full size {w}")
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    z = host(ws.transpose_read(dev["dy"], dev["g"], dev["x"], dev["eta"], dev["alpha"],
                               dev["W0"]))
    for b, h in ((0, 0), (7, 15)):
        sl = lambda k: inp[k][b:b + 1, h:h + 1]  # noqa: E731
        want = oracle.qkv_fwd(sl("dy"), sl("g"), sl("x"), sl("eta"), sl("alpha"),
                              inp["W0"][h:h + 1].transpose(0, 2, 1))
        err = relmax(z[b, h], want[0, 0])
        assert err <= TOL["bf16"], (b, h, err)


@pytest.mark.parametrize("io,bound", [("f64", 1e-12), ("f32", 1e-4)])
def test_two_layer_mechanism_and_control(io, bound):
    # the pages' mechanism test, read with two linear adapted layers: given
    # the serial learner's costates, the forward scans reproduce its outputs,
    # and the transpose read through the adapted second layer reproduces its
    # hidden costates; the control reads through W2^T (eta = 0: D stays zero)
    # and misses them by a large margin while the outputs are unchanged
    T, d0, d1, d2 = 300, 32, 64, 48
    say(f"two-layer mechanism io={io} T={T} d={d0},{d1},{d2}")
    rng = np.random.default_rng(1800)
    X = round_to(rng.standard_normal((1, 1, T, d0)) / np.sqrt(d0), io)
    R = round_to(rng.standard_normal((1, 1, T, d2)), io)
    W1 = round_to(rng.standard_normal((1, d1, d0)) / np.sqrt(d0), io)
    W2 = round_to(rng.standard_normal((1, d2, d1)) / np.sqrt(d1), io)
    gate = "f64" if io == "f64" else "f32"
    e1 = round_to(np.full((1, 1, T), 0.05), gate)
    e2 = round_to(np.full((1, 1, T), 0.08), gate)
    a1 = round_to(np.full((1, 1, T), 0.97), gate)
    a2 = round_to(np.full((1, 1, T), 0.95), gate)
    Hs, Y, G1, G2 = oracle.serial_two_layer(X[0, 0], R[0, 0], e1[0, 0], a1[0, 0], W1[0],
                                            e2[0, 0], a2[0, 0], W2[0])
    tio, tg = TORCH_IO[io], TORCH_IO[gate]
    D = lambda A, t=tio: torch.from_numpy(np.ascontiguousarray(A)).to("cuda", t)  # noqa: E731
    h, _ = ws.gl_scan_fwd(D(X), D(G1[None, None]), D(e1, tg), D(a1, tg), D(W1), save=False)
    y, _ = ws.gl_scan_fwd(h, D(G2[None, None]), D(e2, tg), D(a2, tg), D(W2), save=False)
    g2, _, _ = ws.gl_costate_quadratic(y, D(R), D(G2[None, None]))
    g1 = ws.transpose_read(g2, D(G2[None, None]), h, D(e2, tg), D(a2, tg), D(W2))
    g1c = ws.transpose_read(g2, D(G2[None, None]), h, D(np.zeros_like(e2), tg), D(a2, tg), D(W2))
    torch.cuda.synchronize()
    scale = max(float(np.max(np.abs(G1))), 1.0)
    err_y = np.max(np.abs(host(y)[0, 0] - Y)) / max(float(np.max(np.abs(Y))), 1.0)
    err_g1 = np.max(np.abs(host(g1)[0, 0] - G1)) / scale
    err_ctrl = np.max(np.abs(host(g1c)[0, 0] - G1)) / scale
    say(f"  outputs {err_y:.3g}  hidden costates {err_g1:.3g}  control {err_ctrl:.3g}")
    assert err_y <= bound and err_g1 <= bound
    assert err_ctrl > 1e-2
