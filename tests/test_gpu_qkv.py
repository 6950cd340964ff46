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
