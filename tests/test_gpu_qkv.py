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


@pytest.mark.parametrize("T", [1, 63, 65, 300, 1100])  # 1100: groups of 8, 8 and 2 chunks
@pytest.mark.parametrize("transposed", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_on_the_matrix_cores(d, T, transposed):
    # bf16 with dk = dv = 64 runs the forward matrix-core kernel with a read
    # tile of its own, dk = dv = 128 the state pass and the chunk-parallel
    # outputs (with the workspace the binding passes); GL_FLAG_GENERIC keeps
    # both on the token-serial kernel.  Every route within the scan's bf16
    # bounds of the oracle (max-norm and the RMS / bias / slope statistics).
    from parity_util import error_stats, stats_ok
    say(f"bf16 d={d} matrix cores T={T} transposed={transposed}")
    inp, dev = case("bf16", 2, 3, T, d, d, seed=1900 + T + int(transposed) + d)
    rng = np.random.default_rng(1950 + T)
    qn = round_to(rng.standard_normal(inp["x"].shape) / 8.0, "bf16")
    qd = torch.from_numpy(qn).to("cuda", torch.bfloat16)
    W0p = np.ascontiguousarray(np.transpose(inp["W0"], (0, 2, 1))) if transposed else inp["W0"]
    want = oracle.qkv_fwd(qn, inp["g"], inp["x"], inp["eta"], inp["alpha"], W0p)
    for flags in (0, ws.GL_FLAG_GENERIC):
        y = ws.gl_scan_qkv_fwd(qd, dev["g"], dev["x"], dev["eta"], dev["alpha"], dev["W0"],
                               w0_transposed=transposed, flags=flags)
        torch.cuda.synchronize()
        err = relmax(host(y), want)
        st = error_stats(host(y), want)
        say(f"  flags {flags}: relmax {err:.3g} {st}")
        assert err <= TOL["bf16"], (flags, err)
        assert stats_ok(st), (flags, st)


def test_transpose_read_full_size_sampled_d128():
    # the 1.3B-model shape (B=4, H=16, T=4096, d=128, bf16) on the matrix
    # cores, three heads against the oracle
    w = CONFIGS["c4"]
    say(f"transpose read full size {w}")
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    z = host(ws.transpose_read(dev["dy"], dev["g"], dev["x"], dev["eta"], dev["alpha"],
                               dev["W0"]))
    for b, h in ((0, 0), (2, 9), (3, 15)):
        sl = lambda k: inp[k][b:b + 1, h:h + 1]  # noqa: E731
        want = oracle.qkv_fwd(sl("dy"), sl("g"), sl("x"), sl("eta"), sl("alpha"),
                              inp["W0"][h:h + 1].transpose(0, 2, 1))
        err = relmax(z[b, h], want[0, 0])
        assert err <= TOL["bf16"], (b, h, err)


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
    Hs, Y, G1, G2, GW1 = oracle.serial_two_layer(X[0, 0], R[0, 0], e1[0, 0], a1[0, 0], W1[0],
                                            e2[0, 0], a2[0, 0], W2[0])
    tio, tg = TORCH_IO[io], TORCH_IO[gate]
    D = lambda A, t=tio: torch.from_numpy(np.ascontiguousarray(A)).to("cuda", t)  # noqa: E731
    h, _ = ws.gl_scan_fwd(D(X), D(G1[None, None]), D(e1, tg), D(a1, tg), D(W1), save=False)
    y, _ = ws.gl_scan_fwd(h, D(G2[None, None]), D(e2, tg), D(a2, tg), D(W2), save=False)
    g2, _, _ = ws.gl_costate_quadratic(y, D(R), D(G2[None, None]))
    g1 = ws.transpose_read(g2, D(G2[None, None]), h, D(e2, tg), D(a2, tg), D(W2))
    g1c = ws.transpose_read(g2, D(G2[None, None]), h, D(np.zeros_like(e2), tg), D(a2, tg), D(W2))
    # the first matrix's gradient: the first layer's reverse scan driven by
    # the reconstructed hidden costates (dW0 of gl_scan_bwd with dy = g1)
    xs, g1s = D(X), D(G1[None, None])
    dW1 = ws.gl_scan_bwd(xs, g1s, D(e1, tg), D(a1, tg), D(W1), g1, None)[4]
    dW1c = ws.gl_scan_bwd(xs, g1s, D(e1, tg), D(a1, tg), D(W1), g1c, None)[4]
    torch.cuda.synchronize()
    scale = max(float(np.max(np.abs(G1))), 1.0)
    err_y = np.max(np.abs(host(y)[0, 0] - Y)) / max(float(np.max(np.abs(Y))), 1.0)
    err_g1 = np.max(np.abs(host(g1)[0, 0] - G1)) / scale
    err_ctrl = np.max(np.abs(host(g1c)[0, 0] - G1)) / scale
    sw = max(float(np.max(np.abs(GW1))), 1.0)
    err_w = np.max(np.abs(host(dW1)[0] - GW1)) / sw
    err_wc = np.max(np.abs(host(dW1c)[0] - GW1)) / sw
    say(f"  outputs {err_y:.3g}  hidden costates {err_g1:.3g}  first-matrix gradient "
        f"{err_w:.3g}; control: hidden costates {err_ctrl:.3g}, first-matrix gradient {err_wc:.3g}")
    assert err_y <= bound and err_g1 <= bound and err_w <= bound
    assert err_ctrl > 1e-2 and err_wc > 1e-2


QKV_BWD = [
    ("f64", 2, 2, 70, 16, 16, False),
    ("f32", 1, 2, 150, 64, 48, False),
    ("bf16", 1, 2, 200, 128, 128, False),
    ("f32", 1, 1, 77, 100, 37, True),      # ragged dk, dv; W0 given transposed
    ("bf16", 1, 1, 5, 1, 3, False),
    ("f64", 1, 2, 33, 7, 40, True),
]


@pytest.mark.parametrize("io,B,H,T,dk,dv,w0t", QKV_BWD)
def test_qkv_bwd_parity(io, B, H, T, dk, dv, w0t):
    say(f"qkv backward io={io} B={B} H={H} T={T} dk={dk} dv={dv} w0t={w0t}")
    w = Workload("qkvb", B, H, T, dk, dv, io, "mix", "gauss", 1900 + dk + dv)
    inp = make_inputs(w)
    rng = np.random.default_rng(1950 + T)
    q = round_to(rng.standard_normal(inp["x"].shape) / np.sqrt(dk), io)
    W0p = inp["W0"]                                      # [H, dv, dk]
    W0g = np.ascontiguousarray(W0p.transpose(0, 2, 1)) if w0t else W0p
    dev = to_device(inp, io)
    qd = torch.from_numpy(q).to("cuda", TORCH_IO[io])
    W0d = torch.from_numpy(W0g).to("cuda", TORCH_IO[io])
    got = ws.gl_scan_qkv_bwd(qd, dev["x"], dev["g"], dev["eta"], dev["alpha"], W0d, dev["dy"],
                             w0_transposed=w0t)
    torch.cuda.synchronize()
    want = oracle.qkv_bwd(q, inp["x"], inp["g"], inp["eta"], inp["alpha"], W0p, inp["dy"])
    want = list(want)
    if w0t:
        want[5] = want[5].transpose(0, 2, 1)
    errs = {n: relmax(host(gv), wv) for n, gv, wv in
            zip(("dq", "dk", "dv", "deta", "dalpha", "dW0"), got, want)}
    say(f"  errs {errs}")
    bad = {n: e for n, e in errs.items() if not e <= TOL[io]}
    assert not bad, errs


@pytest.mark.parametrize("d,B,H,T,w0t", [
    (64, 1, 2, 200, False),       # three full chunks and a ragged one
    (64, 2, 1, 129, True),        # one token past two chunks; W0 given transposed
    (64, 1, 1, 64, False),        # exactly one chunk
    (64, 1, 3, 1, True),
    (64, 3, 2, 320, True),        # five full chunks
    (64, 1, 1, 1100, False),      # 18 chunks: three groups of eight, the last ragged
    (128, 1, 2, 200, False),      # W0 transposed by the library
    (128, 2, 1, 129, True),
    (128, 1, 1, 64, True),
    (128, 1, 2, 1, False),
    (128, 1, 1, 1100, True),
])
def test_qkv_bwd_bf16_on_the_matrix_cores(d, B, H, T, w0t):
    # bf16 with dk = dv in {64, 128} takes the chunk-parallel matrix-core
    # reverse scan; against the oracle, and against the vector kernels
    # (GL_FLAG_GENERIC)
    say(f"qkv backward matrix cores d={d} B={B} H={H} T={T} w0t={w0t}")
    w = Workload("qkvb", B, H, T, d, d, "bf16", "mix", "gauss", 2100 + T + d)
    inp = make_inputs(w)
    rng = np.random.default_rng(2150 + T)
    q = round_to(rng.standard_normal(inp["x"].shape) / np.sqrt(d), "bf16")
    W0p = inp["W0"]
    W0g = np.ascontiguousarray(W0p.transpose(0, 2, 1)) if w0t else W0p
    dev = to_device(inp, "bf16")
    qd = torch.from_numpy(q).to("cuda", torch.bfloat16)
    W0d = torch.from_numpy(W0g).to("cuda", torch.bfloat16)
    args = (qd, dev["x"], dev["g"], dev["eta"], dev["alpha"], W0d, dev["dy"])
    got = ws.gl_scan_qkv_bwd(*args, w0_transposed=w0t)
    gen = ws.gl_scan_qkv_bwd(*args, w0_transposed=w0t, flags=ws.GL_FLAG_GENERIC)
    torch.cuda.synchronize()
    want = list(oracle.qkv_bwd(q, inp["x"], inp["g"], inp["eta"], inp["alpha"], W0p, inp["dy"]))
    if w0t:
        want[5] = want[5].transpose(0, 2, 1)
    from parity_util import error_stats, stats_ok
    names = ("dq", "dk", "dv", "deta", "dalpha", "dW0")
    errs = {n: relmax(host(gv), wv) for n, gv, wv in zip(names, got, want)}
    errg = {n: relmax(host(gv), host(hv)) for n, gv, hv in zip(names, got, gen)}
    stats = {n: error_stats(host(gv), wv) for n, gv, wv in zip(names, got, want)}
    say(f"  vs oracle {errs}\n  vs vector kernels {errg}\n  statistics {stats}")
    assert all(e <= TOL["bf16"] for e in errs.values()), errs
    assert all(e <= TOL["bf16"] for e in errg.values()), errg
    # the scan's bf16 RMS / bias / slope bounds for every gradient
    assert all(stats_ok(st) for st in stats.values()), stats


@pytest.mark.parametrize("cfg", ["c3", "c4"])
def test_qkv_bwd_transpose_read_full_size_sampled(cfg):
    # the transpose read's reverse scan at the 340M- and 1.3B-model shapes,
    # every head on the GPU, two heads against the oracle
    w = CONFIGS[cfg]
    say(f"qkv backward full size {w}")
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    # transpose read: q = u (the dy draw), k = g, v = x, W0 given transposed
    rng = np.random.default_rng(1990)
    dz = round_to(rng.standard_normal(inp["x"].shape), w.dtype)
    dzd = torch.from_numpy(dz).to("cuda", TORCH_IO[w.dtype])
    got = ws.gl_scan_qkv_bwd(dev["dy"], dev["g"], dev["x"], dev["eta"], dev["alpha"], dev["W0"],
                             dzd, w0_transposed=True)
    got = [host(t) for t in got]
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = lambda a: a[b:b + 1, h:h + 1]  # noqa: E731
        want = oracle.qkv_bwd(sl(inp["dy"]), sl(inp["g"]), sl(inp["x"]), sl(inp["eta"]),
                              sl(inp["alpha"]), inp["W0"][h:h + 1].transpose(0, 2, 1), sl(dz))
        for n, gv, wv in zip(("dq", "dk", "dv", "deta", "dalpha"), got, want):
            err = relmax(gv[b, h], wv[0, 0])
            assert err <= TOL["bf16"], (b, h, n, err)


@pytest.mark.parametrize("d", [64, 128])
def test_qkv_bwd_matrix_cores_bitwise_repeatable(d):
    # the chunk-parallel reverse scan sums in a fixed order (no atomics): two
    # calls on the same inputs agree bit for bit, W0' plain and transposed
    say(f"qkv backward determinism d={d}")
    w = Workload("qkvd", 2, 2, 700, d, d, "bf16", "mix", "gauss", 2300 + d)
    inp = make_inputs(w)
    dev = to_device(inp, "bf16")
    for w0t in (False, True):
        W0 = dev["W0"].transpose(1, 2).contiguous() if w0t else dev["W0"]
        args = (dev["dy"], dev["g"], dev["x"], dev["eta"], dev["alpha"], W0, dev["dy"])
        first = ws.gl_scan_qkv_bwd(*args, w0_transposed=w0t)
        second = ws.gl_scan_qkv_bwd(*args, w0_transposed=w0t)
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk", "dv", "deta", "dalpha", "dW0"), first, second):
            assert torch.equal(a, b), (w0t, n)
