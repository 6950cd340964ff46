"""Serial fp64 CPU oracle for the GradLev fast-weight scan (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library ``weight_scans_amd`` and never touches a GPU.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one token at a time); this
module only builds it with gcc and marshals numpy arrays.  See ``oracle.h`` for
the recurrence and the page passages it follows.

Parity status of each function: ``fwd`` and ``bwd`` are pinned by the CPU tests
in ``tests/test_oracle.py`` (closed forms, the parallel discounted-sum form,
torch autograd, finite differences, serial-learner recovery, the causal fixed
point and the gate-gradient identity).  ``final_state``, ``decode_readout`` and
``decode_update`` (the serial recurrence of ``seq_fwd`` applied per
sequence-head) are pinned there too: the unrolled discounted sum of the final
adaptation, hand-computed single steps, and a decode loop that reproduces the
whole-sequence readouts.  ``serial_learner`` (the closed-loop learner of the
synthetic test) is pinned by the exact-recovery test (the open-loop C scan
driven by its costates reproduces its outputs, at the rounding scale the
pages print) and the causal fixed-point test; ``costate_quadratic`` by
hand-computed values and by vanishing at the serial learner's costates.
``serial_two_layer`` (two adapted linear layers) is pinned by the open-loop
composition of ``fwd`` and the transpose read of ``qkv_fwd`` driven by its
costates, and its first-matrix gradient by torch autograd through a serial
two-layer loop of the test's own.  ``qkv_bwd`` (the adjoint of ``qkv_fwd``) is
pinned by torch autograd through a serial loop written in the test, central
finite differences, the adjoint dot test, and by reducing to the C oracle's
``bwd`` when q = k = x (dq + dk = dx).  ``qkv_fwd`` (read vector q and write key k of their own) is pinned by
reducing to ``fwd`` when q = k = x, by the transpose read against the
adaptation states of ``seq_fwd``, and by the unrolled discounted sum for a
separate write key.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_seq_fwd.argtypes = [i64, i64, i64] + [p] * 8
        lib.oracle_seq_fwd.restype = None
        lib.oracle_seq_bwd.argtypes = [i64, i64, i64] + [p] * 6 + [i64, i32] + [p] * 5
        lib.oracle_seq_bwd.restype = None
        lib.oracle_fwd.argtypes = [i64] * 5 + [p] * 6 + [i32]
        lib.oracle_fwd.restype = None
        lib.oracle_bwd.argtypes = [i64] * 5 + [p] * 6 + [i64, i32] + [p] * 5 + [i32]
        lib.oracle_bwd.restype = None
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def fwd(x, g, eta, alpha, W0, nthreads: int = 1):
    """y[B,H,T,d_out] = serial readout of the adapted map (fp64)."""
    x, g, eta, alpha, W0 = map(_f64, (x, g, eta, alpha, W0))
    B, H, T, d_in = x.shape
    d_out = g.shape[-1]
    assert g.shape == (B, H, T, d_out) and eta.shape == (B, H, T)
    assert alpha.shape == (B, H, T) and W0.shape == (H, d_out, d_in)
    y = np.empty((B, H, T, d_out), np.float64)
    _load().oracle_fwd(B, H, T, d_in, d_out, _ptr(x), _ptr(g), _ptr(eta),
                       _ptr(alpha), _ptr(W0), _ptr(y), int(nthreads))
    return y


def bwd(x, g, eta, alpha, W0, dy, nthreads: int = 1, ckpt: int = 256,
        variant: int = 0):
    """(dx, dg, deta, dalpha, dW0) of L = sum <dy, y> by the serial adjoint.

    ``variant=1`` is the page's negative control (W0^T instead of the adapted
    transpose in the input gradient); it exists only for the mutation test.
    """
    x, g, eta, alpha, W0, dy = map(_f64, (x, g, eta, alpha, W0, dy))
    B, H, T, d_in = x.shape
    d_out = g.shape[-1]
    assert dy.shape == g.shape and W0.shape == (H, d_out, d_in)
    dx = np.empty_like(x)
    dg = np.empty_like(g)
    deta = np.empty_like(eta)
    dalpha = np.empty_like(alpha)
    dW0 = np.empty_like(W0)
    _load().oracle_bwd(B, H, T, d_in, d_out, _ptr(x), _ptr(g), _ptr(eta),
                       _ptr(alpha), _ptr(W0), _ptr(dy), int(ckpt), int(variant),
                       _ptr(dx), _ptr(dg), _ptr(deta), _ptr(dalpha), _ptr(dW0),
                       int(nthreads))
    return dx, dg, deta, dalpha, dW0


def seq_fwd(x, g, eta, alpha, W0, S_init=None):
    """One sequence: returns (y[T,d_out], D_T[d_out,d_in])."""
    x, g, eta, alpha, W0 = map(_f64, (x, g, eta, alpha, W0))
    T, d_in = x.shape
    d_out = g.shape[-1]
    y = np.empty((T, d_out), np.float64)
    S = np.empty((d_out, d_in), np.float64)
    Si = _f64(S_init) if S_init is not None else None
    _load().oracle_seq_fwd(T, d_in, d_out, _ptr(x), _ptr(g), _ptr(eta),
                           _ptr(alpha), _ptr(W0), _ptr(Si), _ptr(y), _ptr(S))
    return y, S


def final_state(x, g, eta, alpha):
    """Adaptation after the last token of every sequence-head, from zero
    ([B,H,T,d] inputs -> [B,H,d_out,d_in]); the serial recurrence with W0 = 0."""
    x, g, eta, alpha = map(_f64, (x, g, eta, alpha))
    B, H, T, d_in = x.shape
    d_out = g.shape[-1]
    out = np.empty((B, H, d_out, d_in), np.float64)
    Wz = np.zeros((d_out, d_in), np.float64)
    for b in range(B):
        for h in range(H):
            _, out[b, h] = seq_fwd(x[b, h], g[b, h], eta[b, h], alpha[b, h], Wz)
    return out


def decode_readout(x1, W0, S):
    """One token against the cached adaptation S: y = (W0 + S) x
    (x1 [B,H,d_in], W0 [H,d_out,d_in], S [B,H,d_out,d_in] -> [B,H,d_out])."""
    x1, W0, S = map(_f64, (x1, W0, S))
    B, H, d_in = x1.shape
    d_out = W0.shape[1]
    y = np.empty((B, H, d_out), np.float64)
    for b in range(B):
        for h in range(H):
            yt, _ = seq_fwd(x1[b, h][None], np.zeros((1, d_out)), np.zeros(1), np.ones(1),
                            W0[h], S_init=S[b, h])
            y[b, h] = yt[0]
    return y


def decode_update(x1, g1, eta1, alpha1, S):
    """One step of the recurrence on the cached adaptation: returns
    alpha S - eta g x^T (x1 [B,H,d_in], g1 [B,H,d_out], eta1/alpha1 [B,H])."""
    x1, g1, eta1, alpha1, S = map(_f64, (x1, g1, eta1, alpha1, S))
    B, H, d_in = x1.shape
    d_out = g1.shape[-1]
    out = np.empty_like(S)
    Wz = np.zeros((d_out, d_in), np.float64)
    for b in range(B):
        for h in range(H):
            _, out[b, h] = seq_fwd(x1[b, h][None], g1[b, h][None], eta1[b, h][None],
                                   alpha1[b, h][None], Wz, S_init=S[b, h])
    return out


def serial_learner(X, R, eta, alpha, W0):
    """The ordinary serial learner of one sequence-head under the quadratic
    token loss |y_t - r_t|^2 / 2 ("Parallelize the Training, Keep the Learning
    Serial", section "The synthetic test checks the mechanism, not model
    quality"): each token reads out from the current weight, takes its own
    costate g_t = y_t - r_t and updates at once.  Returns (Y [T,d_out],
    G [T,d_out])."""
    X, R, eta, alpha, W0 = map(_f64, (X, R, eta, alpha, W0))
    D = np.zeros_like(W0)
    Y = np.empty((X.shape[0], W0.shape[0]))
    G = np.empty_like(Y)
    for t in range(X.shape[0]):
        Y[t] = (W0 + D) @ X[t]
        G[t] = Y[t] - R[t]
        D = alpha[t] * D - eta[t] * np.outer(G[t], X[t])
    return Y, G


def costate_quadratic(y, target, g_hat):
    """Reconstructed costates under the quadratic token loss and the
    consistency residual per token (section "The predictor is constrained by
    the learner it is supposed to reproduce"): g~ = y - target,
    res_sq = sum_r (g^ - g~)^2, res_max = max_r |g^ - g~|."""
    y, target, g_hat = map(_f64, (y, target, g_hat))
    g_tilde = y - target
    e = g_hat - g_tilde
    return g_tilde, np.sum(e * e, axis=-1), np.max(np.abs(e), axis=-1, initial=0.0)


def qkv_fwd(q, k, v, eta, alpha, W0p):
    """The scan with its own read vector and write key, token by token:
    y_t = (W0' + D_t) q_t, D_{t+1} = alpha_t D_t - eta_t v_t k_t^T, D_0 = 0
    (q, k [B,H,T,dk], v [B,H,T,dv], W0p [H,dv,dk] -> y [B,H,T,dv]).  With
    q = k = x, v = g it is the forward scan; with q = u, k = g, v = x and
    W0p = W0^T the transpose read (W0 + D_t)^T u_t ("Parallelize the Training,
    Keep the Learning Serial", section "The synthetic test checks the
    mechanism, not model quality")."""
    q, k, v, eta, alpha, W0p = map(_f64, (q, k, v, eta, alpha, W0p))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    y = np.empty((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            D = np.zeros((dv, dk))
            for t in range(T):
                y[b, h, t] = (W0p[h] + D) @ q[b, h, t]
                D = alpha[b, h, t] * D - eta[b, h, t] * np.outer(v[b, h, t], k[b, h, t])
    return y


def qkv_bwd(q, k, v, eta, alpha, W0p, dy, ckpt: int = 64):
    """The exact adjoint of qkv_fwd for L = sum_t <dy_t, y_t>, token by token
    in reverse ("Parallelize the Training, Keep the Learning Serial", section
    "Once the gradient signals are known, the weight trajectory becomes
    parallelizable": the recurrence is affine in D, so its adjoint is the same
    recurrence run backwards).  With A the adjoint of the adaptation written
    by token t (A = 0 after the last token):
        dq_t = (W0' + D_t)^T dy_t        dk_t = -eta_t A^T v_t
        dv_t = -eta_t A k_t              deta_t = -v_t^T A k_t
        dalpha_t = <A, D_t>              dW0' += dy_t q_t^T
        A <- alpha_t A + dy_t q_t^T
    D_t is kept every `ckpt` tokens and recomputed forward within a block.
    Returns (dq, dk, dv, deta, dalpha, dW0p) with dW0p [H,dv,dk] summed over
    the batch."""
    q, k, v, eta, alpha, W0p, dy = map(_f64, (q, k, v, eta, alpha, W0p, dy))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dq, dkk = np.zeros_like(q), np.zeros_like(k)
    dvv = np.zeros_like(v)
    deta, dalpha = np.zeros_like(eta), np.zeros_like(alpha)
    dW0p = np.zeros_like(W0p)
    for b in range(B):
        for h in range(H):
            qs, ks, vs = q[b, h], k[b, h], v[b, h]
            es, al, g = eta[b, h], alpha[b, h], dy[b, h]
            # forward: the adaptation read by token t, kept at block starts
            marks = {}
            D = np.zeros((dv, dk))
            for t in range(T):
                if t % ckpt == 0:
                    marks[t] = D.copy()
                D = al[t] * D - es[t] * np.outer(vs[t], ks[t])
            A = np.zeros((dv, dk))
            for t0 in range(((T - 1) // ckpt) * ckpt if T else 0, -1, -ckpt):
                t1 = min(T, t0 + ckpt)
                Ds = [marks[t0]]
                for t in range(t0, t1 - 1):
                    Ds.append(al[t] * Ds[-1] - es[t] * np.outer(vs[t], ks[t]))
                for t in range(t1 - 1, t0 - 1, -1):
                    Dt = Ds[t - t0]
                    dq[b, h, t] = (W0p[h] + Dt).T @ g[t]
                    dkk[b, h, t] = -es[t] * (A.T @ vs[t])
                    dvv[b, h, t] = -es[t] * (A @ ks[t])
                    deta[b, h, t] = -vs[t] @ A @ ks[t]
                    dalpha[b, h, t] = np.sum(A * Dt)
                    dW0p[h] += np.outer(g[t], qs[t])
                    A = al[t] * A + np.outer(g[t], qs[t])
    return dq, dkk, dvv, deta, dalpha, dW0p


def serial_two_layer(X, R, eta1, alpha1, W1, eta2, alpha2, W2):
    """The serial learner of the two-layer synthetic test ("Parallelize the
    Training, Keep the Learning Serial", section "The synthetic test checks the
    mechanism, not model quality"), read with both layers linear and adapted:
    h_t = W1_{t-1} x_t, y_t = W2_{t-1} h_t, g2_t = y_t - r_t, the hidden
    costate g1_t = W2_{t-1}^T g2_t (through the weight that produced y_t), then
    both layers take their step.  Returns (H, Y, G1, G2, GW1): GW1 is the
    first matrix's gradient, the sum over tokens of the test-time gradients
    d l_t / d W1 = g1_t x_t^T taken at each token's weights (with the
    costates held as data it is the gradient of sum_t l_t w.r.t. the
    persistent W1)."""
    X, R, eta1, alpha1, W1, eta2, alpha2, W2 = map(
        _f64, (X, R, eta1, alpha1, W1, eta2, alpha2, W2))
    T = X.shape[0]
    D1 = np.zeros_like(W1)
    D2 = np.zeros_like(W2)
    Hs = np.empty((T, W1.shape[0]))
    Y = np.empty((T, W2.shape[0]))
    G1, G2 = np.empty_like(Hs), np.empty_like(Y)
    GW1 = np.zeros_like(W1)
    for t in range(T):
        Hs[t] = (W1 + D1) @ X[t]
        Y[t] = (W2 + D2) @ Hs[t]
        G2[t] = Y[t] - R[t]
        G1[t] = (W2 + D2).T @ G2[t]
        GW1 += np.outer(G1[t], X[t])
        D2 = alpha2[t] * D2 - eta2[t] * np.outer(G2[t], Hs[t])
        D1 = alpha1[t] * D1 - eta1[t] * np.outer(G1[t], X[t])
    return Hs, Y, G1, G2, GW1
