"""weight_scans_amd: GradLev fast-weight scans on MI355X (HIP, gfx950).

All arithmetic runs in the HIP shared library ``libglscan.so`` behind the C ABI
of ``include/gl_scan.h``.  This module only marshals torch tensors (device
memory and the current stream) into those calls; it has no compute fallback and
raises if the library is missing.

    y, saved = gl_scan_fwd(x, g, eta, alpha, W0)
    dx, dg, deta, dalpha, dW0 = gl_scan_bwd(x, g, eta, alpha, W0, dy, saved)
    y = scan(x, g, eta, alpha, W0)          # autograd-aware
    state = gl_scan_final_state(x, g, eta, alpha)     # prefill -> decode
    y1 = gl_decode_readout(x1, W0, state)             # one token
    gl_decode_update(x1, g1, eta1, alpha1, state)     # in place
    y2 = gl_decode_step(x1, g1, eta1, alpha1, x2, W0, state)  # both, fused
    g_t, res_sq, res_max = gl_costate_quadratic(y, target, g_hat)  # quadratic loss
    g, y, sweeps = picard(x, eta, alpha, W0, target)   # fixed point of g -> g~
    y = gl_scan_qkv_fwd(q, k, v, eta, alpha, W0)       # read vector != write key
    dq, dk, dv, deta, dalpha, dW0 = gl_scan_qkv_bwd(q, k, v, eta, alpha, W0, dy)
    z = transpose_read(u, g, x, eta, alpha, W0)       # (W0 + D_t)^T u_t

Shapes: x [B,H,T,d_in], g [B,H,T,d_out], eta/alpha [B,H,T], W0 [H,d_out,d_in];
one decode token: x1 [B,H,d_in], g1 [B,H,d_out], eta1/alpha1 [B,H];
state [B,H,d_out,d_in] in the gate dtype.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libglscan.so")

EXPORTS = (
    "gl_scan_saved_size",
    "gl_scan_workspace_size",
    "gl_scan_fwd",
    "gl_scan_bwd",
    "gl_status_string",
    "gl_last_error",
    "gl_scan_path_name",
    "gl_decode_readout",
    "gl_decode_update",
    "gl_decode_step",
    "gl_scan_final_state",
    "gl_costate_quadratic",
    "gl_scan_qkv_fwd",
    "gl_scan_qkv_workspace_size",
    "gl_scan_qkv_bwd",
    "gl_scan_bwd_static",
    "gl_scan_qkv_fwd_workspace_size",
    "gl_scan_qkv_fwd_ws",
)

GL_FLAG_GENERIC = 1
GL_FLAG_OUT_F32 = 2
GL_DTYPE_F64, GL_DTYPE_F32, GL_DTYPE_BF16 = 0, 1, 2
STATUS_NAMES = {0: "GL_SUCCESS", 1: "GL_ERROR_INVALID_VALUE", 2: "GL_ERROR_NOT_SUPPORTED",
                3: "GL_ERROR_MISALIGNED", 4: "GL_ERROR_WORKSPACE_TOO_SMALL", 5: "GL_ERROR_HIP"}


class GLScanError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("segments", ctypes.c_uint32)]


_lib = None


def lib():
    """Load libglscan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m weight_scans_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        pd = ctypes.POINTER(Desc)
        ps = ctypes.POINTER(ctypes.c_size_t)
        L.gl_scan_saved_size.argtypes = [pd, ps]
        L.gl_scan_workspace_size.argtypes = [pd, I, ps, ps]
        L.gl_scan_fwd.argtypes = [pd] + [P] * 7 + [P, S, P]
        L.gl_scan_bwd.argtypes = [pd] + [P] * 12 + [P, S, P]
        L.gl_decode_readout.argtypes = [pd] + [P] * 5
        L.gl_decode_update.argtypes = [pd] + [P] * 6
        L.gl_scan_final_state.argtypes = [pd] + [P] * 6
        L.gl_decode_step.argtypes = [pd] + [P] * 9
        L.gl_costate_quadratic.argtypes = [pd] + [P] * 7
        L.gl_scan_qkv_fwd.argtypes = [pd] + [P] * 6 + [I] + [P] * 2
        L.gl_scan_qkv_workspace_size.argtypes = [pd, ps]
        L.gl_scan_bwd_static.argtypes = [pd] + [P] * 12 + [P]
        L.gl_scan_qkv_bwd.argtypes = [pd] + [P] * 6 + [I] + [P] * 7 + [P, S, P]
        L.gl_scan_qkv_fwd_workspace_size.argtypes = [pd, ps]
        L.gl_scan_qkv_fwd_ws.argtypes = [pd] + [P] * 6 + [I, P, P, S, P]
        for f in ("gl_scan_saved_size", "gl_scan_workspace_size", "gl_scan_fwd", "gl_scan_bwd",
                  "gl_decode_readout", "gl_decode_update", "gl_decode_step",
                  "gl_scan_final_state", "gl_costate_quadratic", "gl_scan_qkv_fwd",
                  "gl_scan_qkv_workspace_size", "gl_scan_qkv_bwd", "gl_scan_bwd_static",
                  "gl_scan_qkv_fwd_workspace_size", "gl_scan_qkv_fwd_ws"):
            getattr(L, f).restype = ctypes.c_int
        L.gl_status_string.argtypes = [I]
        L.gl_status_string.restype = ctypes.c_char_p
        L.gl_last_error.argtypes = []
        L.gl_last_error.restype = ctypes.c_char_p
        L.gl_scan_path_name.argtypes = [pd]
        L.gl_scan_path_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise GLScanError(status, lib().gl_last_error().decode())


def make_desc(B, H, T, d_in, d_out, io_dtype, chunk=0, flags=0, segments=0) -> Desc:
    """segments: 0 = automatic, 1 = none, n = n segments per sequence."""
    return Desc(B, H, T, d_in, d_out, io_dtype, chunk, flags, segments)


def path_name(desc: Desc) -> str | None:
    r = lib().gl_scan_path_name(ctypes.byref(desc))
    return r.decode() if r else None


def saved_size(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib().gl_scan_saved_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def workspace_size(desc: Desc, have_saved: bool):
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().gl_scan_workspace_size(ctypes.byref(desc), int(have_saved),
                                        ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


# ---------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _io_code(dtype):
    torch = _torch()
    return {torch.float64: GL_DTYPE_F64, torch.float32: GL_DTYPE_F32,
            torch.bfloat16: GL_DTYPE_BF16}[dtype]


def gate_dtype(io_dtype):
    torch = _torch()
    return torch.float64 if io_dtype == torch.float64 else torch.float32


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _validate(x, g, eta, alpha, W0, dy=None):
    if x.dim() != 4 or g.dim() != 4:
        raise ValueError("x and g must be [B,H,T,d]")
    B, H, T, d_in = x.shape
    d_out = g.shape[-1]
    gd = gate_dtype(x.dtype)
    if g.shape[:3] != (B, H, T) or tuple(W0.shape) != (H, d_out, d_in):
        raise ValueError("shape mismatch between x, g and W0")
    if eta.shape != (B, H, T) or alpha.shape != (B, H, T):
        raise ValueError("eta/alpha must be [B,H,T]")
    if dy is not None and dy.shape != g.shape:
        raise ValueError("dy must have the shape of g")
    for t in (x, g, W0) + ((dy,) if dy is not None else ()):
        if t.dtype != x.dtype:
            raise TypeError("x, g, W0 and dy must share the io dtype")
    for t in (eta, alpha):
        if t.dtype != gd:
            raise TypeError(f"eta/alpha must be {gd}")
    for t in (x, g, eta, alpha, W0) + ((dy,) if dy is not None else ()):
        if not t.is_cuda:
            raise ValueError("all tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    return B, H, T, d_in, d_out


def _out_dtype(io_dtype, flags):
    """dtype of y, dx and dg: fp32 for bf16 io under GL_FLAG_OUT_F32."""
    torch = _torch()
    if (flags & GL_FLAG_OUT_F32) and io_dtype == torch.bfloat16:
        return torch.float32
    return io_dtype


def gl_scan_fwd(x, g, eta, alpha, W0, *, chunk=0, flags=0, save=True, segments=0):
    """Forward scan.  Returns (y, saved) where saved is None if save=False."""
    torch = _torch()
    B, H, T, d_in, d_out = _validate(x, g, eta, alpha, W0)
    desc = make_desc(B, H, T, d_in, d_out, _io_code(x.dtype), chunk, flags, segments)
    y = torch.empty((B, H, T, d_out), dtype=_out_dtype(x.dtype, flags), device=x.device)
    saved = None
    if save:
        saved = torch.empty(max(saved_size(desc), 16), dtype=torch.uint8, device=x.device)
    fws, _ = workspace_size(desc, save)
    ws = torch.empty(max(fws, 16), dtype=torch.uint8, device=x.device)
    _check(lib().gl_scan_fwd(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(eta), _ptr(alpha),
                             _ptr(W0), _ptr(y), _ptr(saved), _ptr(ws), fws,
                             _stream(x.device)))
    return y, saved


def gl_scan_bwd(x, g, eta, alpha, W0, dy, saved=None, *, chunk=0, flags=0, segments=0):
    """Reverse scan.  Returns (dx, dg, deta, dalpha, dW0)."""
    torch = _torch()
    B, H, T, d_in, d_out = _validate(x, g, eta, alpha, W0, dy)
    desc = make_desc(B, H, T, d_in, d_out, _io_code(x.dtype), chunk, flags, segments)
    gd = gate_dtype(x.dtype)
    od = _out_dtype(x.dtype, flags)
    dx = torch.empty(x.shape, dtype=od, device=x.device)
    dg = torch.empty(g.shape, dtype=od, device=x.device)
    deta = torch.empty_like(eta)
    dalpha = torch.empty_like(alpha)
    dW0 = torch.empty((H, d_out, d_in), dtype=gd, device=x.device)
    _, bws = workspace_size(desc, saved is not None)
    ws = torch.empty(max(bws, 16), dtype=torch.uint8, device=x.device)
    _check(lib().gl_scan_bwd(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(eta), _ptr(alpha),
                             _ptr(W0), _ptr(dy), _ptr(saved), _ptr(dx), _ptr(dg), _ptr(deta),
                             _ptr(dalpha), _ptr(dW0), _ptr(ws), bws, _stream(x.device)))
    return dx, dg, deta, dalpha, dW0


def gl_scan_bwd_static(x, g, eta, alpha, W0, dy, saved=None, *, chunk=0, flags=0, segments=0,
                       out=None):
    """gl_scan_bwd through the no-allocation entry point (the library's static
    scratch, no workspace).  `out` may hold preallocated (dx, dg, deta, dalpha,
    dW0); returns them."""
    torch = _torch()
    B, H, T, d_in, d_out = _validate(x, g, eta, alpha, W0, dy)
    desc = make_desc(B, H, T, d_in, d_out, _io_code(x.dtype), chunk, flags, segments)
    if out is None:
        gd = gate_dtype(x.dtype)
        od = _out_dtype(x.dtype, flags)
        out = (torch.empty(x.shape, dtype=od, device=x.device),
               torch.empty(g.shape, dtype=od, device=x.device),
               torch.empty_like(eta), torch.empty_like(alpha),
               torch.empty((H, d_out, d_in), dtype=gd, device=x.device))
    dx, dg, deta, dalpha, dW0 = out
    _check(lib().gl_scan_bwd_static(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(eta),
                                    _ptr(alpha), _ptr(W0), _ptr(dy), _ptr(saved), _ptr(dx),
                                    _ptr(dg), _ptr(deta), _ptr(dalpha), _ptr(dW0),
                                    _stream(x.device)))
    return dx, dg, deta, dalpha, dW0


def _check_dec(tensors, gates, state, io_dtype):
    gd = gate_dtype(io_dtype)
    for t in tensors:
        if t.dtype != io_dtype:
            raise TypeError("x, g and W0 must share the io dtype")
    for t in gates + (state,):
        if t.dtype != gd:
            raise TypeError(f"eta/alpha/state must be {gd}")
    for t in tensors + gates + (state,):
        if not t.is_cuda:
            raise ValueError("all tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def gl_scan_final_state(x, g, eta, alpha, flags=0):
    """Adaptation after the last of T prefill tokens, [B,H,d_out,d_in]
    (flags=GL_FLAG_GENERIC: fp32 vector arithmetic for the matrix-core shapes)."""
    torch = _torch()
    if x.dim() != 4 or g.dim() != 4:
        raise ValueError("x and g must be [B,H,T,d]")
    B, H, T, d_in = x.shape
    d_out = g.shape[-1]
    if g.shape[:3] != (B, H, T) or eta.shape != (B, H, T) or alpha.shape != (B, H, T):
        raise ValueError("shape mismatch between x, g, eta and alpha")
    state = torch.empty((B, H, d_out, d_in), dtype=gate_dtype(x.dtype), device=x.device)
    _check_dec((x, g), (eta, alpha), state, x.dtype)
    desc = make_desc(B, H, T, d_in, d_out, _io_code(x.dtype), flags=flags)
    _check(lib().gl_scan_final_state(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(eta),
                                     _ptr(alpha), _ptr(state), _stream(x.device)))
    return state


def gl_decode_readout(x, W0, state, y=None):
    """y = (W0 + state) x for one token; x [B,H,d_in] -> y [B,H,d_out]."""
    torch = _torch()
    if x.dim() != 3 or state.dim() != 4:
        raise ValueError("x must be [B,H,d_in] and state [B,H,d_out,d_in]")
    B, H, d_in = x.shape
    d_out = state.shape[2]
    if tuple(state.shape) != (B, H, d_out, d_in) or tuple(W0.shape) != (H, d_out, d_in):
        raise ValueError("shape mismatch between x, W0 and state")
    if y is None:
        y = torch.empty((B, H, d_out), dtype=x.dtype, device=x.device)
    elif tuple(y.shape) != (B, H, d_out):
        raise ValueError("y must be [B,H,d_out]")
    _check_dec((x, W0, y), (), state, x.dtype)
    desc = make_desc(B, H, 1, d_in, d_out, _io_code(x.dtype))
    _check(lib().gl_decode_readout(ctypes.byref(desc), _ptr(x), _ptr(W0), _ptr(state), _ptr(y),
                                   _stream(x.device)))
    return y


def gl_decode_update(x, g, eta, alpha, state):
    """state <- alpha state - eta g x^T in place for one token; returns state."""
    if x.dim() != 3 or g.dim() != 3 or state.dim() != 4:
        raise ValueError("x, g must be [B,H,d] and state [B,H,d_out,d_in]")
    B, H, d_in = x.shape
    d_out = g.shape[-1]
    if (g.shape[:2] != (B, H) or tuple(state.shape) != (B, H, d_out, d_in)
            or eta.shape != (B, H) or alpha.shape != (B, H)):
        raise ValueError("shape mismatch between x, g, eta, alpha and state")
    _check_dec((x, g), (eta, alpha), state, x.dtype)
    desc = make_desc(B, H, 1, d_in, d_out, _io_code(x.dtype))
    _check(lib().gl_decode_update(ctypes.byref(desc), _ptr(x), _ptr(g), _ptr(eta), _ptr(alpha),
                                  _ptr(state), _stream(x.device)))
    return state


def gl_decode_step(x_prev, g_prev, eta_prev, alpha_prev, x, W0, state, y=None):
    """Update of the previous token, then readout of x; state in place.
    Returns y [B,H,d_out]."""
    torch = _torch()
    if x.dim() != 3 or x_prev.shape != x.shape or state.dim() != 4:
        raise ValueError("x, x_prev must be [B,H,d_in] and state [B,H,d_out,d_in]")
    B, H, d_in = x.shape
    d_out = state.shape[2]
    if (tuple(state.shape) != (B, H, d_out, d_in) or tuple(W0.shape) != (H, d_out, d_in)
            or tuple(g_prev.shape) != (B, H, d_out) or eta_prev.shape != (B, H)
            or alpha_prev.shape != (B, H)):
        raise ValueError("shape mismatch between the step's tensors")
    if y is None:
        y = torch.empty((B, H, d_out), dtype=x.dtype, device=x.device)
    elif tuple(y.shape) != (B, H, d_out):
        raise ValueError("y must be [B,H,d_out]")
    _check_dec((x_prev, g_prev, x, W0, y), (eta_prev, alpha_prev), state, x.dtype)
    desc = make_desc(B, H, 1, d_in, d_out, _io_code(x.dtype))
    _check(lib().gl_decode_step(ctypes.byref(desc), _ptr(x_prev), _ptr(g_prev), _ptr(eta_prev),
                                _ptr(alpha_prev), _ptr(x), _ptr(W0), _ptr(state), _ptr(y),
                                _stream(x.device)))
    return y


def gl_costate_quadratic(y, target, g_hat, g_tilde=None):
    """Reconstructed costates g~ = y - target and the per-token consistency
    residuals (|g^ - g~|^2, max |g^ - g~|) for the quadratic token loss."""
    torch = _torch()
    if y.dim() != 4 or target.shape != y.shape or g_hat.shape != y.shape:
        raise ValueError("y, target and g_hat must be [B,H,T,d_out] of one shape")
    B, H, T, d_out = y.shape
    if g_tilde is None:
        g_tilde = torch.empty_like(y)
    elif g_tilde.shape != y.shape:
        raise ValueError("g_tilde must have the shape of y")
    gd = gate_dtype(y.dtype)
    res_sq = torch.empty((B, H, T), dtype=gd, device=y.device)
    res_max = torch.empty((B, H, T), dtype=gd, device=y.device)
    _check_dec((y, target, g_hat, g_tilde), (res_sq, res_max), res_max, y.dtype)
    desc = make_desc(B, H, T, 1, d_out, _io_code(y.dtype))
    _check(lib().gl_costate_quadratic(ctypes.byref(desc), _ptr(y), _ptr(target), _ptr(g_hat),
                                      _ptr(g_tilde), _ptr(res_sq), _ptr(res_max),
                                      _stream(y.device)))
    return g_tilde, res_sq, res_max


def picard(x, eta, alpha, W0, target, g0=None, max_sweeps=None, tol=0.0):
    """Picard iteration of the causal costate map for the quadratic token loss:
    g <- y(g) - target, y(g) = gl_scan_fwd(x, g, ...), from g0 (zero by
    default), until the largest residual is <= tol or max_sweeps (default T)
    sweeps have run.  Returns (g, y, sweeps, res_max of the last sweep)."""
    torch = _torch()
    B, H, T, _ = x.shape
    g = torch.zeros_like(target) if g0 is None else g0.clone()
    g_next = torch.empty_like(g)
    n = T if max_sweeps is None else max_sweeps
    y, res_max, k = None, None, 0
    for k in range(1, n + 1):
        y, _ = gl_scan_fwd(x, g, eta, alpha, W0, save=False)
        _, _, res_max = gl_costate_quadratic(y, target, g, g_tilde=g_next)
        g, g_next = g_next, g
        if float(res_max.max()) <= tol:
            break
    return g, y, k, res_max


def gl_scan_qkv_fwd(q, k, v, eta, alpha, W0, w0_transposed=False, flags=0):
    """y_t = (W0' + D_t) q_t, D_{t+1} = alpha_t D_t - eta_t v_t k_t^T: q, k
    [B,H,T,dk], v [B,H,T,dv], W0 [H,dv,dk] (or [H,dk,dv] transposed).
    flags: GL_FLAG_GENERIC keeps bf16 d = 64 off the matrix cores."""
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    want = (H, dk, dv) if w0_transposed else (H, dv, dk)
    if tuple(W0.shape) != want or eta.shape != (B, H, T) or alpha.shape != (B, H, T):
        raise ValueError("shape mismatch between q, v, W0, eta and alpha")
    y = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check_dec((q, k, v, W0, y), (eta,), alpha, q.dtype)
    desc = make_desc(B, H, T, dk, dv, _io_code(q.dtype), flags=flags)
    n = ctypes.c_size_t()
    _check(lib().gl_scan_qkv_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=q.device) if n.value else None
    _check(lib().gl_scan_qkv_fwd_ws(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                    _ptr(alpha), _ptr(W0), int(bool(w0_transposed)), _ptr(y),
                                    _ptr(ws), n.value, _stream(q.device)))
    return y


def gl_scan_qkv_bwd(q, k, v, eta, alpha, W0, dy, w0_transposed=False, flags=0):
    """Reverse scan of gl_scan_qkv_fwd for upstream dy [B,H,T,dv].  Returns
    (dq, dk, dv, deta, dalpha, dW0) with dW0 in the layout W0 is given in.
    flags: GL_FLAG_GENERIC keeps bf16 d = 64 off the matrix cores."""
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dvv = v.shape[-1]
    want = (H, dk, dvv) if w0_transposed else (H, dvv, dk)
    if (tuple(W0.shape) != want or eta.shape != (B, H, T) or alpha.shape != (B, H, T)
            or dy.shape != v.shape):
        raise ValueError("shape mismatch between q, v, W0, eta, alpha and dy")
    gd = gate_dtype(q.dtype)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    deta, dalpha = torch.empty_like(eta), torch.empty_like(alpha)
    dW0 = torch.empty(want, dtype=gd, device=q.device)
    _check_dec((q, k, v, W0, dy, dq, dk_, dv_), (eta, deta, dalpha), alpha, q.dtype)
    desc = make_desc(B, H, T, dk, dvv, _io_code(q.dtype), flags=flags)
    n = ctypes.c_size_t()
    _check(lib().gl_scan_qkv_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=q.device)
    _check(lib().gl_scan_qkv_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                 _ptr(alpha), _ptr(W0), int(bool(w0_transposed)), _ptr(dy),
                                 _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(deta), _ptr(dalpha),
                                 _ptr(dW0), _ptr(ws), n.value, _stream(q.device)))
    return dq, dk_, dv_, deta, dalpha, dW0


def transpose_read(u, g, x, eta, alpha, W0, flags=0):
    """z_t = (W0 + D_t)^T u_t along the adaptation D_t that (x, g, eta, alpha)
    write (u [B,H,T,d_out] -> z [B,H,T,d_in])."""
    return gl_scan_qkv_fwd(u, g, x, eta, alpha, W0, w0_transposed=True, flags=flags)


def _make_function():
    torch = _torch()

    class ScanFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, g, eta, alpha, W0, chunk, flags):
            y, saved = gl_scan_fwd(x, g, eta, alpha, W0, chunk=chunk, flags=flags)
            ctx.save_for_backward(x, g, eta, alpha, W0, saved)
            ctx.chunk, ctx.flags = chunk, flags
            return y

        @staticmethod
        def backward(ctx, dy):
            x, g, eta, alpha, W0, saved = ctx.saved_tensors
            dx, dg, deta, dalpha, dW0 = gl_scan_bwd(x, g, eta, alpha, W0, dy.contiguous(),
                                                    saved, chunk=ctx.chunk, flags=ctx.flags)
            return dx, dg, deta, dalpha, dW0.to(W0.dtype), None, None

    return ScanFunction


_fn = None


def scan(x, g, eta, alpha, W0, chunk=0, flags=0):
    """Autograd-aware forward scan y = scan(x, g, eta, alpha, W0)."""
    global _fn
    if _fn is None:
        _fn = _make_function()
    return _fn.apply(x, g, eta, alpha, W0, chunk, flags)
