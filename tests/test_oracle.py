"""Pins for the fp64 CPU oracle (no GPU).

Every test here checks the oracle against something other than its own loop:
closed forms, the parallel discounted-sum form of the weight correction, torch
autograd, finite differences, exact recovery of the closed-loop serial learner,
the causal fixed point and a gate-gradient identity.  Page references are to
"Parallelize the Training, Keep the Learning Serial" (cognaptus.com) unless
stated otherwise.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from weight_scans_amd.synth import Workload, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "recovery_magnitudes.txt")


def small(B=1, H=1, T=16, d_in=8, d_out=8, seed=7, alpha="base", x="gauss"):
    w = Workload("t", B, H, T, d_in, d_out, "f64", alpha, x, seed)
    return make_inputs(w)


def relmax(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def run_both(inp, **kw):
    y = oracle.fwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"])
    grads = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"],
                       inp["dy"], **kw)
    return y, grads


# ---------------------------------------------------------------------------
# Independent parallel (closed) form: the adaptation is a discounted sum of the
# earlier rank-one updates (section "Once the gradient signals are known, the
# weight trajectory becomes parallelizable").  With V = -diag(eta) G and
# M[i, j] = prod_{r=j+1}^{i-1} alpha_r for j < i (else 0):
#   y  = X W0^T + (M o X X^T) V
# and the adjoint of that dense expression, derived by hand:
#   dV = (M o XX^T)^T dY,  dg = -eta dV,  deta = -rowsum(G o dV)
#   E  = M o (dY V^T),     dX = dY W0 + E X + E^T X,   dW0 = dY^T X
#   dlog(alpha_r) = sum_{j < r < i} (M o XX^T o dY V^T)[i, j]
# ---------------------------------------------------------------------------
def decay_matrix(alpha):
    T = len(alpha)
    M = np.zeros((T, T))
    for i in range(T):
        p = 1.0
        for j in range(i - 1, -1, -1):
            M[i, j] = p
            p *= alpha[j]
    return M


def parallel_form(x, g, eta, alpha, W0, dy):
    X, G, dY = x, g, dy
    M = decay_matrix(alpha)
    V = -eta[:, None] * G
    XX = X @ X.T
    P = M * XX
    y = X @ W0.T + P @ V
    dV = P.T @ dY
    dg = -eta[:, None] * dV
    deta = -np.sum(G * dV, axis=1)
    E = M * (dY @ V.T)
    dX = dY @ W0 + E @ X + E.T @ X
    dW0 = dY.T @ X
    Z = M * XX * (dY @ V.T)
    T = len(alpha)
    dlog = np.zeros(T)
    for r in range(T):
        dlog[r] = Z[r + 1:, :r].sum()
    return y, dX, dg, deta, dlog / alpha, dW0


def test_identity_gates_reduce_to_static_map():
    """alpha = 1, eta = 0: no adaptation, y = W0 x; closed forms for the rest."""
    inp = small(B=2, H=2, T=24, d_in=6, d_out=5, seed=11)
    inp["alpha"][:] = 1.0
    inp["eta"][:] = 0.0
    y, (dx, dg, deta, dal, dW0) = run_both(inp)
    X, G, dY, W0 = inp["x"], inp["g"], inp["dy"], inp["W0"]
    y_ref = np.einsum("hoi,bhti->bhto", W0, X)
    assert relmax(y, y_ref) < 1e-14
    assert relmax(dx, np.einsum("hoi,bhto->bhti", W0, dY)) < 1e-14
    assert np.all(dg == 0.0) and np.all(dal == 0.0)
    assert relmax(dW0, np.einsum("bhto,bhti->hoi", dY, X)) < 1e-14
    # deta_t = -sum_{u > t} (g_t . dy_u)(x_u . x_t)
    gd = np.einsum("bhto,bhuo->bhtu", G, dY)
    xx = np.einsum("bhui,bhti->bhtu", X, X)
    strict_upper = np.triu(np.ones((24, 24)), k=1)
    deta_ref = -np.sum(gd * xx * strict_upper, axis=-1)
    assert relmax(deta, deta_ref) < 1e-13


def test_structural_zeros():
    """D_0 = 0 gives dalpha_0 = 0; the last update is never read, so
    deta, dg and dalpha vanish at t = T-1."""
    inp = small(B=2, H=3, T=37, d_in=5, d_out=7, seed=3)
    _, (dx, dg, deta, dal, dW0) = run_both(inp)
    assert np.all(dal[..., 0] == 0.0)
    assert np.all(deta[..., -1] == 0.0)
    assert np.all(dg[..., -1, :] == 0.0)
    assert np.all(dal[..., -1] == 0.0)


def test_first_two_tokens_by_hand():
    """y_0 = W0 x_0 and y_1 = W0 x_1 - eta_0 (x_0 . x_1) g_0; neither depends
    on any alpha (alpha_0 multiplies the zero adaptation)."""
    inp = small(T=2, d_in=4, d_out=3, seed=5)
    X, G, e, W0 = inp["x"][0, 0], inp["g"][0, 0], inp["eta"][0, 0], inp["W0"][0]
    y = oracle.fwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"])[0, 0]
    assert relmax(y[0], W0 @ X[0]) < 1e-15
    assert relmax(y[1], W0 @ X[1] - e[0] * (X[0] @ X[1]) * G[0]) < 1e-15
    inp2 = dict(inp)
    inp2["alpha"] = np.full_like(inp["alpha"], 0.123)
    y2 = oracle.fwd(inp2["x"], inp2["g"], inp2["eta"], inp2["alpha"], inp2["W0"])[0, 0]
    assert np.array_equal(y, y2)
    # T = 1: a single readout from W0
    one = small(T=1, d_in=4, d_out=3, seed=9)
    y1, (dx1, dg1, de1, da1, dW1) = run_both(one)
    assert relmax(y1[0, 0, 0], one["W0"][0] @ one["x"][0, 0, 0]) < 1e-15
    assert np.all(dg1 == 0) and np.all(de1 == 0) and np.all(da1 == 0)


@pytest.mark.parametrize("seed,alpha", [(21, "base"), (22, "mix"), (23, "near1")])
def test_parallel_discounted_sum_form(seed, alpha):
    """Serial loop vs the dense parallel form (forward and all gradients)."""
    inp = small(T=48, d_in=7, d_out=6, seed=seed, alpha=alpha)
    y, (dx, dg, deta, dal, dW0) = run_both(inp)
    ref = parallel_form(*(inp[k][0, 0] if k != "W0" else inp[k][0]
                          for k in ("x", "g", "eta", "alpha", "W0", "dy")))
    for got, want in zip((y[0, 0], dx[0, 0], dg[0, 0], deta[0, 0], dal[0, 0], dW0[0]), ref):
        assert relmax(got, want) < 1e-12


def _torch_serial(x, g, eta, alpha, W0):
    D = torch.zeros_like(W0)
    ys = []
    for t in range(x.shape[0]):
        ys.append((W0 + D) @ x[t])
        D = alpha[t] * D - eta[t] * torch.outer(g[t], x[t])
    return torch.stack(ys)


def test_torch_autograd_small():
    """Brute-force autodiff (torch fp64 CPU) through the serial loop."""
    inp = small(B=1, H=1, T=14, d_in=6, d_out=5, seed=31, alpha="mix")
    names = ("x", "g", "eta", "alpha")
    tens = {k: torch.tensor(inp[k][0, 0], requires_grad=True) for k in names}
    W0 = torch.tensor(inp["W0"][0], requires_grad=True)
    y = _torch_serial(tens["x"], tens["g"], tens["eta"], tens["alpha"], W0)
    (y * torch.tensor(inp["dy"][0, 0])).sum().backward()
    _, (dx, dg, deta, dal, dW0) = run_both(inp)
    assert relmax(dx[0, 0], tens["x"].grad.numpy()) < 1e-13
    assert relmax(dg[0, 0], tens["g"].grad.numpy()) < 1e-13
    assert relmax(deta[0, 0], tens["eta"].grad.numpy()) < 1e-13
    assert relmax(dal[0, 0], tens["alpha"].grad.numpy()) < 1e-13
    assert relmax(dW0[0], W0.grad.numpy()) < 1e-13


def test_central_finite_differences():
    inp = small(B=1, H=1, T=6, d_in=3, d_out=4, seed=41)
    _, grads = run_both(inp)
    names = ("x", "g", "eta", "alpha", "W0")
    h = 1e-6

    def f(d):
        y = oracle.fwd(d["x"], d["g"], d["eta"], d["alpha"], d["W0"])
        return float(np.sum(y * d["dy"]))

    for name, grad in zip(names, (grads[0], grads[1], grads[2], grads[3], grads[4])):
        fd = np.zeros_like(inp[name])
        for idx in np.ndindex(inp[name].shape):
            p = {k: v.copy() for k, v in inp.items()}
            m = {k: v.copy() for k, v in inp.items()}
            p[name][idx] += h
            m[name][idx] -= h
            fd[idx] = (f(p) - f(m)) / (2 * h)
        assert np.max(np.abs(fd - grad)) < 1e-8, name


def test_adjoint_dot_product():
    """<grad, v> equals the directional derivative along a random v."""
    inp = small(B=2, H=2, T=120, d_in=12, d_out=10, seed=51, alpha="mix")
    _, grads = run_both(inp)
    names = ("x", "g", "eta", "alpha", "W0")
    rng = np.random.default_rng(0)
    v = {k: rng.standard_normal(inp[k].shape) for k in names}
    eps = 1e-5

    def f(s):
        d = dict(inp)
        for k in names:
            d[k] = inp[k] + s * v[k]
        y = oracle.fwd(d["x"], d["g"], d["eta"], d["alpha"], d["W0"])
        return float(np.sum(y * inp["dy"]))

    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = sum(float(np.sum(gr * v[k])) for k, gr in zip(names, grads))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def _golden():
    vals = {}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def test_exact_recovery_of_serial_learner():
    """Supplying the serial learner's own costates G* to the open-loop scan
    reproduces its outputs, and the costates reconstructed from those outputs
    equal G*, at rounding scale (section "The synthetic test checks the
    mechanism, not model quality": ~1e-16 discrepancies)."""
    inp = small(T=200, d_in=16, d_out=16, seed=61, alpha="mix")
    X, eta, alpha, W0 = inp["x"][0, 0], inp["eta"][0, 0], inp["alpha"][0, 0], inp["W0"][0]
    R = np.random.default_rng(62).standard_normal((200, 16))
    Y_star, G_star = oracle.serial_learner(X, R, eta, alpha, W0)
    y = oracle.fwd(X[None, None], G_star[None, None], eta[None, None],
                   alpha[None, None], W0[None])[0, 0]
    g_rec = y - R
    page = _golden()
    scale = max(np.max(np.abs(Y_star)), 1.0)
    err_y = np.max(np.abs(y - Y_star)) / scale
    err_g = np.max(np.abs(g_rec - G_star)) / scale
    # rounding scale: within two orders of the largest printed discrepancy
    bound = 100 * max(page["outputs"], page["hidden_costates"], page["first_matrix_gradients"])
    assert err_y < bound and err_g < bound


def test_causal_fixed_point_iteration():
    """The costate map is causal: g~_t depends only on g^_{<t}.  Picard
    iteration from zero fixes one more token per sweep and reaches the serial
    learner's costates after T sweeps (section "The predictor is constrained
    by the learner it is supposed to reproduce")."""
    T = 12
    inp = small(T=T, d_in=5, d_out=5, seed=71, alpha="base")
    X, eta, alpha, W0 = inp["x"][0, 0], inp["eta"][0, 0], inp["alpha"][0, 0], inp["W0"][0]
    inp["eta"][:] = 0.5  # strong coupling so that the iterates really differ
    eta = inp["eta"][0, 0]
    R = np.random.default_rng(72).standard_normal((T, 5))
    _, G_star = oracle.serial_learner(X, R, eta, alpha, W0)
    G = np.zeros_like(G_star)
    for k in range(1, T + 1):
        y = oracle.fwd(X[None, None], G[None, None], eta[None, None],
                       alpha[None, None], W0[None])[0, 0]
        G = y - R
        assert np.max(np.abs(G[:k] - G_star[:k])) < 1e-12
        if k <= 4:
            # not yet fixed: the next token still carries the earlier error
            assert np.max(np.abs(G[k] - G_star[k])) > 1e-9
    assert np.max(np.abs(G - G_star)) < 1e-12


def test_gate_gradient_identity():
    """dalpha_r alpha_r = sum_{t>r} q_t - sum_{s>=r} k_s with
    q_t = dy_t . (y_t - W0 x_t) and k_s = eta_s deta_s: the oracle's direct
    <Lambda, D> form agrees with a form built from its other outputs."""
    inp = small(B=2, H=2, T=90, d_in=9, d_out=7, seed=81, alpha="mix")
    y, (dx, dg, deta, dal, dW0) = run_both(inp)
    q = np.einsum("bhto,bhto->bht", inp["dy"],
                  y - np.einsum("hoi,bhti->bhto", inp["W0"], inp["x"]))
    k = inp["eta"] * deta
    suf_q = np.flip(np.cumsum(np.flip(q, -1), -1), -1)   # sum_{t >= r}
    suf_k = np.flip(np.cumsum(np.flip(k, -1), -1), -1)
    rhs = (suf_q - q) - suf_k
    assert relmax(dal * inp["alpha"], rhs) < 1e-11


def test_segment_composition_and_checkpoints_are_exact():
    """Associativity in practice: running [0, T1) then [T1, T) from the handed
    over adaptation equals one run; the backward's checkpoint interval and the
    thread count do not change a single bit."""
    inp = small(B=3, H=2, T=77, d_in=6, d_out=5, seed=91, alpha="mix")
    X, G, e, a, W0 = (inp["x"][1, 1], inp["g"][1, 1], inp["eta"][1, 1],
                      inp["alpha"][1, 1], inp["W0"][1])
    y_full, S_full = oracle.seq_fwd(X, G, e, a, W0)
    y_a, S_a = oracle.seq_fwd(X[:30], G[:30], e[:30], a[:30], W0)
    y_b, S_b = oracle.seq_fwd(X[30:], G[30:], e[30:], a[30:], W0, S_init=S_a)
    assert np.array_equal(np.concatenate([y_a, y_b]), y_full)
    assert np.array_equal(S_b, S_full)
    ref = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], inp["dy"], ckpt=1)
    for ck, nt in ((5, 1), (77, 3), (256, 4)):
        got = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"],
                         inp["dy"], ckpt=ck, nthreads=nt)
        for a_, b_ in zip(got, ref):
            assert np.array_equal(a_, b_)


def test_control_variant_is_caught():
    """The page's negative control (W0^T in place of the adapted transpose in
    the backward) leaves the forward and the other gradients untouched but
    moves the input gradient by O(1) -- the autograd pin detects it."""
    inp = small(B=1, H=1, T=40, d_in=8, d_out=8, seed=101)
    inp["eta"][:] = 0.5
    good = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], inp["dy"])
    bad = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], inp["dy"], variant=1)
    for i in (1, 2, 3, 4):
        assert np.array_equal(good[i], bad[i])
    tx = torch.tensor(inp["x"][0, 0], requires_grad=True)
    y = _torch_serial(tx, torch.tensor(inp["g"][0, 0]), torch.tensor(inp["eta"][0, 0]),
                      torch.tensor(inp["alpha"][0, 0]), torch.tensor(inp["W0"][0]))
    (y * torch.tensor(inp["dy"][0, 0])).sum().backward()
    assert relmax(good[0][0, 0], tx.grad.numpy()) < 1e-13
    page = _golden()
    # same order as the printed control discrepancies (0.3757 / 0.6261)
    assert relmax(bad[0][0, 0], tx.grad.numpy()) > 0.1 * page["control_hidden_costates"]


# ---- deployment: the cached adaptation ("The bottleneck appears before
# deployment"; ParaTTT news summary, section "Perspective")

def test_final_state_is_the_discounted_sum():
    # unrolled: D_T = sum_t (prod_{s>t} alpha_s)(-eta_t) g_t x_t^T
    inp = small(B=2, H=2, T=37, d_in=5, d_out=3, seed=21, alpha="mix")
    got = oracle.final_state(inp["x"], inp["g"], inp["eta"], inp["alpha"])
    a = inp["alpha"]
    suffix = np.concatenate([np.cumprod(a[..., ::-1], axis=-1)[..., ::-1][..., 1:],
                             np.ones(a.shape[:-1] + (1,))], axis=-1)
    w = -suffix * inp["eta"]
    want = np.einsum("bht,bhtr,bhtc->bhrc", w, inp["g"], inp["x"])
    assert relmax(got, want) < 1e-13
    # T = 0: the empty sum; T = 1: one step from zero
    assert np.all(oracle.final_state(inp["x"][:, :, :0], inp["g"][:, :, :0],
                                     inp["eta"][:, :, :0], inp["alpha"][:, :, :0]) == 0)
    one = oracle.final_state(inp["x"][:, :, :1], inp["g"][:, :, :1], inp["eta"][:, :, :1],
                             inp["alpha"][:, :, :1])
    assert np.allclose(one[0, 1], -inp["eta"][0, 1, 0] * np.outer(inp["g"][0, 1, 0],
                                                                    inp["x"][0, 1, 0]))


def test_decode_steps_by_hand():
    S = np.array([[[[1.0, 2.0]]]])        # [B=1,H=1,d_out=1,d_in=2]
    W0 = np.array([[[0.5, 0.5]]])
    x1 = np.array([[[1.0, -1.0]]])
    # (W0 + S) x = 1.5 - 2.5
    assert np.array_equal(oracle.decode_readout(x1, W0, S), np.array([[[-1.0]]]))
    # 0.5 S - 2 * 3 * x^T
    got = oracle.decode_update(x1, np.array([[[3.0]]]), np.array([[2.0]]),
                               np.array([[0.5]]), S)
    assert np.array_equal(got, np.array([[[[-5.5, 7.0]]]]))


def test_decode_loop_reproduces_the_whole_sequence():
    # prefill T0 tokens, hand the adaptation over, decode the rest one at a
    # time: every readout and the last adaptation agree with the whole scan
    inp = small(B=2, H=2, T=50, d_in=6, d_out=4, seed=22)
    T0 = 31
    y_all = oracle.fwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"])
    S = oracle.final_state(*(inp[k][:, :, :T0] for k in ("x", "g", "eta", "alpha")))
    for t in range(T0, 50):
        y_t = oracle.decode_readout(inp["x"][:, :, t], inp["W0"], S)
        assert relmax(y_t, y_all[:, :, t]) < 1e-13
        S = oracle.decode_update(inp["x"][:, :, t], inp["g"][:, :, t], inp["eta"][:, :, t],
                                 inp["alpha"][:, :, t], S)
    want = oracle.final_state(inp["x"], inp["g"], inp["eta"], inp["alpha"])
    assert relmax(S, want) < 1e-13


# ---- costate reconstruction under the quadratic token loss ("The predictor
# is constrained by the learner it is supposed to reproduce")

def test_costate_quadratic_by_hand():
    y = np.array([[[[1.0, -2.0], [0.5, 0.5]]]])       # [1,1,T=2,d=2]
    r = np.array([[[[0.0, -1.0], [1.5, 0.5]]]])
    gh = np.array([[[[1.0, 0.0], [0.0, 0.0]]]])
    gt, sq, mx = oracle.costate_quadratic(y, r, gh)
    assert np.array_equal(gt, np.array([[[[1.0, -1.0], [-1.0, 0.0]]]]))
    # token 0: (0, 1) -> 1, 1; token 1: (1, 0) -> 1, 1
    assert np.array_equal(sq, np.array([[[1.0, 1.0]]]))
    assert np.array_equal(mx, np.array([[[1.0, 1.0]]]))


def test_costate_vanishes_at_the_serial_learner():
    # proposing the serial learner's own costates, the scan reproduces its
    # outputs and the reconstruction returns the proposal: residual ~ 0; a
    # perturbed proposal does not
    inp = small(T=64, d_in=12, d_out=12, seed=91, alpha="mix")
    X, eta, alpha, W0 = inp["x"][0, 0], inp["eta"][0, 0], inp["alpha"][0, 0], inp["W0"][0]
    R = np.random.default_rng(92).standard_normal((64, 12))
    _, G = oracle.serial_learner(X, R, eta, alpha, W0)
    y = oracle.fwd(X[None, None], G[None, None], eta[None, None], alpha[None, None], W0[None])
    gt, sq, mx = oracle.costate_quadratic(y, R[None, None], G[None, None])
    assert np.max(mx) < 1e-12 and np.max(sq) < 1e-24
    G2 = G.copy()
    G2[10] += 0.1
    y2 = oracle.fwd(X[None, None], G2[None, None], eta[None, None], alpha[None, None], W0[None])
    _, _, mx2 = oracle.costate_quadratic(y2, R[None, None], G2[None, None])
    assert mx2[0, 0, 10] > 0.09 and np.max(mx2[0, 0, :10]) < 1e-12  # causal: earlier tokens unmoved


# ---- the scan with its own read vector and write key (transpose read and
# write-key readings; "The synthetic test checks the mechanism, not model
# quality", "Once the gradient signals are known...")

def test_qkv_reduces_to_the_forward_scan():
    inp = small(B=2, H=2, T=40, d_in=6, d_out=5, seed=101, alpha="mix")
    want = oracle.fwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"])
    got = oracle.qkv_fwd(inp["x"], inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"])
    assert relmax(got, want) < 1e-13


def test_transpose_read_against_the_adaptation_states():
    # z_t = (W0 + D_t)^T u_t with D_t taken from the serial recurrence of the
    # C oracle on the prefix [0, t)
    inp = small(T=20, d_in=6, d_out=4, seed=102)
    X, G, e, a = (inp[k][0, 0] for k in ("x", "g", "eta", "alpha"))
    W0 = inp["W0"][0]
    U = np.random.default_rng(103).standard_normal((20, 4))
    z = oracle.qkv_fwd(U[None, None], G[None, None], X[None, None], e[None, None], a[None, None],
                       W0.T[None])[0, 0]
    for t in range(20):
        _, D = oracle.seq_fwd(X[:t], G[:t], e[:t], a[:t], W0)
        assert np.max(np.abs(z[t] - (W0 + D).T @ U[t])) < 1e-13


def test_write_key_closed_form():
    # y_t = W0 x_t + sum_{s<t} (prod_{s<u<t} alpha_u)(-eta_s) g_s (xbar_s . x_t)
    inp = small(T=30, d_in=5, d_out=3, seed=104, alpha="mix")
    X, G, e, a = (inp[k][0, 0] for k in ("x", "g", "eta", "alpha"))
    W0 = inp["W0"][0]
    Xb = X - X.mean(axis=0)  # a centered key
    y = oracle.qkv_fwd(X[None, None], Xb[None, None], G[None, None], e[None, None],
                       a[None, None], W0[None])[0, 0]
    for t in range(30):
        want = W0 @ X[t]
        for s_ in range(t):
            want = want + np.prod(a[s_ + 1:t]) * (-e[s_]) * G[s_] * (Xb[s_] @ X[t])
        assert np.max(np.abs(y[t] - want)) < 1e-13


def test_two_layer_mechanism_and_control():
    # supplied with the serial learner's costates, the open-loop scans
    # reproduce its outputs, and the transpose read through the adapted second
    # layer reproduces its hidden costates at rounding scale; reading through
    # W2^T (the persistent weight) instead leaves the outputs alone but not the
    # hidden costates (the pages' control)
    T, d0, d1, d2 = 60, 6, 8, 5
    rng = np.random.default_rng(111)
    X = rng.standard_normal((T, d0)) / np.sqrt(d0)
    R = rng.standard_normal((T, d2))
    W1 = rng.standard_normal((d1, d0)) / np.sqrt(d0)
    W2 = rng.standard_normal((d2, d1)) / np.sqrt(d1)
    e1, e2 = np.full(T, 0.2), np.full(T, 0.3)
    a1, a2 = np.full(T, 0.95), np.full(T, 0.9)
    Hs, Y, G1, G2, GW1 = oracle.serial_two_layer(X, R, e1, a1, W1, e2, a2, W2)
    b = lambda A: A[None, None]  # noqa: E731
    h = oracle.fwd(b(X), b(G1), b(e1), b(a1), W1[None])[0, 0]
    y = oracle.fwd(b(h), b(G2), b(e2), b(a2), W2[None])[0, 0]
    g2 = y - R
    g1 = oracle.qkv_fwd(b(g2), b(G2), b(h), b(e2), b(a2), W2.T[None])[0, 0]
    g1_ctrl = oracle.qkv_fwd(b(g2), b(G2), b(h), b(np.zeros(T)), b(a2), W2.T[None])[0, 0]
    page = _golden()
    bound = 100 * max(page["outputs"], page["hidden_costates"])
    assert np.max(np.abs(y - Y)) < bound and np.max(np.abs(g1 - G1)) < bound
    assert np.max(np.abs(g1_ctrl - G1)) > 1e-2
    # the first matrix's gradient: the reverse scan of the first layer driven
    # by the reconstructed hidden costates (dW0 of bwd with dy = g1) against
    # the serial learner's sum of per-token gradients; the control's hidden
    # costates move it by O(1)
    dW1 = oracle.bwd(b(X), b(G1), b(e1), b(a1), W1[None], b(g1))[4][0]
    dW1_ctrl = oracle.bwd(b(X), b(G1), b(e1), b(a1), W1[None], b(g1_ctrl))[4][0]
    scale = max(float(np.max(np.abs(GW1))), 1.0)
    assert np.max(np.abs(dW1 - GW1)) / scale < 100 * page["first_matrix_gradients"]
    assert np.max(np.abs(dW1_ctrl - GW1)) / scale > 1e-2


def _torch_two_layer_first_matrix(X, R, e1, a1, W1, e2, a2, W2):
    """Serial autograd of the two-layer learner, written here independently of
    the oracle: at each token the loss |y_t - r_t|^2 / 2 is differentiated by
    torch w.r.t. the first matrix at that token's weights (the adaptations are
    data, detached), the per-token gradients summed; also returns the hidden
    costates dl_t / dh_t."""
    T = X.shape[0]
    W1t, W2t = torch.tensor(W1), torch.tensor(W2)
    D1 = torch.zeros_like(W1t)
    D2 = torch.zeros_like(W2t)
    acc = torch.zeros_like(W1t)
    G1 = []
    for t in range(T):
        A1 = (W1t + D1).clone().requires_grad_(True)
        x = torch.tensor(X[t])
        h = A1 @ x
        h.retain_grad()
        y = (W2t + D2) @ h
        loss = 0.5 * torch.sum((y - torch.tensor(R[t])) ** 2)
        loss.backward()
        acc += A1.grad
        g1, g2 = h.grad.detach(), (y - torch.tensor(R[t])).detach()
        G1.append(g1)
        D2 = a2[t] * D2 - e2[t] * torch.outer(g2, h.detach())
        D1 = a1[t] * D1 - e1[t] * torch.outer(g1, x)
    return acc.numpy(), torch.stack(G1).numpy()


def test_two_layer_first_matrix_gradient_by_autograd():
    T, d0, d1, d2 = 40, 5, 7, 4
    rng = np.random.default_rng(112)
    X = rng.standard_normal((T, d0)) / np.sqrt(d0)
    R = rng.standard_normal((T, d2))
    W1 = rng.standard_normal((d1, d0)) / np.sqrt(d0)
    W2 = rng.standard_normal((d2, d1)) / np.sqrt(d1)
    e1, e2 = np.full(T, 0.15), np.full(T, 0.25)
    a1, a2 = rng.uniform(0.8, 1.0, T), rng.uniform(0.8, 1.0, T)
    _, _, G1, _, GW1 = oracle.serial_two_layer(X, R, e1, a1, W1, e2, a2, W2)
    want, G1t = _torch_two_layer_first_matrix(X, R, e1, a1, W1, e2, a2, W2)
    assert relmax(G1, G1t) < 1e-13
    assert relmax(GW1, want) < 1e-13


# ---- the adjoint of the scan with its own read vector and write key

def _torch_qkv(q, k, v, eta, alpha, W0p):
    T = q.shape[0]
    D = torch.zeros_like(W0p)
    ys = []
    for t in range(T):
        ys.append((W0p + D) @ q[t])
        D = alpha[t] * D - eta[t] * torch.outer(v[t], k[t])
    return torch.stack(ys)


def _qkv_inputs(T, dk, dv, seed, alpha="mix"):
    inp = small(T=T, d_in=dk, d_out=dv, seed=seed, alpha=alpha)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal(inp["x"].shape) / np.sqrt(dk)
    return q, inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"], inp["dy"]


def test_qkv_adjoint_by_torch_autograd():
    q, k, v, e, a, W0, dy = _qkv_inputs(15, 5, 4, 121)
    names = ("q", "k", "v", "eta", "alpha")
    vals = dict(zip(names, (q, k, v, e, a)))
    tens = {n: torch.tensor(vals[n][0, 0], requires_grad=True) for n in names}
    W0t = torch.tensor(W0[0], requires_grad=True)
    y = _torch_qkv(tens["q"], tens["k"], tens["v"], tens["eta"], tens["alpha"], W0t)
    (y * torch.tensor(dy[0, 0])).sum().backward()
    got = oracle.qkv_bwd(q, k, v, e, a, W0, dy, ckpt=4)
    for n, gr in zip(names, got[:5]):
        assert relmax(gr[0, 0], tens[n].grad.numpy()) < 1e-13, n
    assert relmax(got[5][0], W0t.grad.numpy()) < 1e-13


def test_qkv_adjoint_finite_differences():
    q, k, v, e, a, W0, dy = _qkv_inputs(6, 3, 2, 131)
    inp = dict(q=q, k=k, v=v, eta=e, alpha=a, W0=W0)
    got = dict(zip(("q", "k", "v", "eta", "alpha", "W0"),
                   oracle.qkv_bwd(q, k, v, e, a, W0, dy)))
    h = 1e-6

    def f(d):
        y = oracle.qkv_fwd(d["q"], d["k"], d["v"], d["eta"], d["alpha"], d["W0"])
        return float(np.sum(y * dy))

    for name in inp:
        fd = np.zeros_like(inp[name])
        for idx in np.ndindex(inp[name].shape):
            pp = {kk: vv.copy() for kk, vv in inp.items()}
            mm = {kk: vv.copy() for kk, vv in inp.items()}
            pp[name][idx] += h
            mm[name][idx] -= h
            fd[idx] = (f(pp) - f(mm)) / (2 * h)
        assert np.max(np.abs(fd - got[name])) < 1e-8, name


def test_qkv_adjoint_dot_product_and_blocks():
    q, k, v, e, a, W0, dy = _qkv_inputs(150, 9, 7, 141)
    g1 = oracle.qkv_bwd(q, k, v, e, a, W0, dy, ckpt=64)
    g2 = oracle.qkv_bwd(q, k, v, e, a, W0, dy, ckpt=1)   # every state kept
    for x1, x2 in zip(g1, g2):
        assert np.array_equal(x1, x2)
    names = ("q", "k", "v", "eta", "alpha", "W0")
    base = dict(zip(names, (q, k, v, e, a, W0)))
    rng = np.random.default_rng(1)
    dirs = {n: rng.standard_normal(base[n].shape) for n in names}
    eps = 1e-5

    def f(sc):
        d = {n: base[n] + sc * dirs[n] for n in names}
        return float(np.sum(oracle.qkv_fwd(d["q"], d["k"], d["v"], d["eta"], d["alpha"],
                                           d["W0"]) * dy))

    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = sum(float(np.sum(gr * dirs[n])) for n, gr in zip(names, g1))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_qkv_adjoint_reduces_to_the_scan_adjoint():
    # q = k = x, v = g: dq + dk is the C oracle's dx, the rest coincide
    inp = small(B=2, H=2, T=70, d_in=6, d_out=5, seed=151, alpha="mix")
    dx, dg, de, da, dW = oracle.bwd(inp["x"], inp["g"], inp["eta"], inp["alpha"], inp["W0"],
                                    inp["dy"])
    dq, dk, dv, de2, da2, dW2 = oracle.qkv_bwd(inp["x"], inp["x"], inp["g"], inp["eta"],
                                               inp["alpha"], inp["W0"], inp["dy"])
    assert relmax(dq + dk, dx) < 1e-12
    assert relmax(dv, dg) < 1e-12
    assert relmax(de2, de) < 1e-12 and relmax(da2, da) < 1e-12 and relmax(dW2, dW) < 1e-12
