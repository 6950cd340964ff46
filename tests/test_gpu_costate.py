"""GPU-vs-oracle parity of costate reconstruction under the quadratic token
loss and its Picard sweeps, through the C ABI (needs an MI355X).

Tolerances (relative-max error, as in parity_util):
  g~       fp64 1e-10; fp32 1e-6 (one rounding of y - r); bf16 1e-2 (g~ is
           rounded to bf16: 2^-9 relative)
  res_sq   1e-10 (fp64), 1e-4 (fp32 arithmetic over d_out <= 128 terms)
  res_max  1e-10 (fp64), 1e-5
  Picard   the scan's own tolerance (fp64 1e-10, fp32 1e-4, bf16 2e-2)
"""
import numpy as np
import pytest
import torch

import oracle
import weight_scans_amd as ws
from parity_util import TOL, TORCH_IO, host, relmax, to_device
from weight_scans_amd.synth import Workload, make_inputs, round_to

pytestmark = pytest.mark.gpu

G_TOL = {"f64": 1e-10, "f32": 1e-6, "bf16": 1e-2}
SQ_TOL = {"f64": 1e-10, "f32": 1e-4, "bf16": 1e-4}
MX_TOL = {"f64": 1e-10, "f32": 1e-5, "bf16": 1e-5}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    ws.lib()


@pytest.mark.parametrize("io,B,H,T,d", [
    ("f64", 2, 3, 100, 64),
    ("f32", 1, 2, 77, 100),          # no vector layout: lanes stride the row
    ("bf16", 2, 2, 300, 128),
    ("f32", 1, 1, 5, 1),
    ("bf16", 8, 16, 4096, 64),       # the 340M-model shape, every token
])
def test_costate_parity(io, B, H, T, d):
    say(f"costate io={io} B={B} H={H} T={T} d={d}")
    w = Workload("cost", B, H, T, d, d, io, "base", "gauss", 1100 + d)
    inp = make_inputs(w)
    target = round_to(np.random.default_rng(1200 + d).standard_normal((B, H, T, d)), io)
    tio = TORCH_IO[io]
    y = torch.from_numpy(inp["dy"]).to("cuda", tio)
    gh = torch.from_numpy(inp["g"]).to("cuda", tio)
    r = torch.from_numpy(target).to("cuda", tio)
    gt, sq, mx = ws.gl_costate_quadratic(y, r, gh)
    torch.cuda.synchronize()
    w_gt, w_sq, w_mx = oracle.costate_quadratic(inp["dy"], target, inp["g"])
    e = (relmax(host(gt), w_gt), relmax(host(sq), w_sq), relmax(host(mx), w_mx))
    assert e[0] <= G_TOL[io] and e[1] <= SQ_TOL[io] and e[2] <= MX_TOL[io], e


def picard_case(io, B, H, T, d, seed):
    w = Workload("picard", B, H, T, d, d, io, "base", "gauss", seed)
    inp = make_inputs(w)
    R = round_to(np.random.default_rng(seed + 1).standard_normal((B, H, T, d)), io)
    dev = to_device(inp, io)
    dev["R"] = torch.from_numpy(R).to("cuda", TORCH_IO[io])
    G = np.empty((B, H, T, d))
    for b in range(B):
        for h in range(H):
            _, G[b, h] = oracle.serial_learner(inp["x"][b, h], R[b, h], inp["eta"][b, h],
                                               inp["alpha"][b, h], inp["W0"][h])
    return dev, G


@pytest.mark.parametrize("io,T,d", [("f64", 40, 16), ("f32", 150, 64), ("bf16", 200, 64),
                                    ("bf16", 130, 128)])
def test_picard_reaches_the_serial_learner(io, T, d):
    # sweeps of (scan, reconstruction) from zero costates converge to the
    # costates of the serial learner (the unique fixed point of the causal map)
    say(f"picard io={io} T={T} d={d}")
    dev, G = picard_case(io, 1, 2, T, d, seed=1300 + d)
    g, _, sweeps, res = ws.picard(dev["x"], dev["eta"], dev["alpha"], dev["W0"], dev["R"],
                                  max_sweeps=T, tol=0.0 if io == "f64" else 1e-6)
    torch.cuda.synchronize()
    err = relmax(host(g), G)
    say(f"  sweeps={sweeps} last res_max={float(res.max()):.3g} err={err:.3g}")
    assert err <= TOL[io], err


def test_picard_fixes_one_more_token_per_sweep():
    # causality: after k sweeps from zero the first k tokens are exact, and
    # with strong coupling the next token is not yet
    io, T, d = "f64", 24, 8
    dev, G = picard_case(io, 1, 1, T, d, seed=1400)
    dev["eta"].fill_(0.5)
    eta = host(dev["eta"])
    inp_x, W0 = host(dev["x"]), host(dev["W0"])
    _, G = oracle.serial_learner(inp_x[0, 0], host(dev["R"])[0, 0], eta[0, 0],
                                 host(dev["alpha"])[0, 0], W0[0])
    for k in (1, 3, 6):
        g, _, _, _ = ws.picard(dev["x"], dev["eta"], dev["alpha"], dev["W0"], dev["R"],
                               max_sweeps=k)
        gk = host(g)[0, 0]
        assert np.max(np.abs(gk[:k] - G[:k])) < 1e-10
        assert np.max(np.abs(gk[k] - G[k])) > 1e-8


def test_empty_is_a_noop():
    y = torch.empty((2, 0, 5, 8), dtype=torch.float32, device="cuda")
    gt, sq, mx = ws.gl_costate_quadratic(y, y, y)
    assert gt.shape == y.shape and sq.shape == (2, 0, 5)
