"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything (the
pointers passed here are never dereferenced)."""
import ctypes
import os
import re

import pytest

import weight_scans_amd as ws

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "gl_scan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gl_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(ws.EXPORTS) == declared_functions()


def test_library_exports_every_declared_symbol():
    L = ws.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def desc(**kw):
    base = dict(B=2, H=3, T=100, d_in=64, d_out=64, io_dtype=ws.GL_DTYPE_BF16, chunk=0, flags=0)
    base.update(kw)
    return ws.make_desc(**base)


def status(fn, *args):
    return getattr(ws.lib(), fn)(*args)


def test_status_strings():
    L = ws.lib()
    for code in range(6):
        assert L.gl_status_string(code)
    assert L.gl_status_string(99) == b"unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 1), (dict(T=-5), 1), (dict(d_in=0), 1), (dict(io_dtype=7), 1),
    (dict(flags=8), 1), (dict(chunk=-1), 1),
    (dict(d_in=129), 2), (dict(d_out=256), 2), (dict(chunk=48), 2),
    (dict(io_dtype=ws.GL_DTYPE_F64, chunk=32), 2),
    (dict(segments=1 << 21), 1), (dict(io_dtype=ws.GL_DTYPE_F32, segments=2), 2),
    (dict(flags=ws.GL_FLAG_GENERIC, segments=3), 2),
    (dict(chunk=128), 2), (dict(io_dtype=ws.GL_DTYPE_F32, chunk=128), 2),
    (dict(io_dtype=ws.GL_DTYPE_F64, chunk=128), 2), (dict(chunk=24), 2),
    (dict(io_dtype=ws.GL_DTYPE_F64, flags=ws.GL_FLAG_OUT_F32), 2),
    (dict(flags=4), 1),
    (dict(io_dtype=ws.GL_DTYPE_F32, d_in=100, chunk=64), 2),
    (dict(io_dtype=ws.GL_DTYPE_F64, chunk=64), 2),
    (dict(io_dtype=ws.GL_DTYPE_F32, segments=3), 2),
])
def test_descriptor_validation(kw, code):
    d = desc(**kw)
    n = ctypes.c_size_t()
    assert ws.lib().gl_scan_saved_size(ctypes.byref(d), ctypes.byref(n)) == code
    assert ws.path_name(d) is None


@pytest.mark.parametrize("kw,path", [
    (dict(), "mfma-bf16-d64"), (dict(chunk=64), "mfma-bf16-d64"),
    (dict(chunk=16), "generic-bf16"), (dict(chunk=32), "generic-bf16"),
    (dict(flags=ws.GL_FLAG_OUT_F32), "mfma-bf16-d64"),
    (dict(flags=ws.GL_FLAG_OUT_F32 | ws.GL_FLAG_GENERIC), "generic-bf16-out-f32"),
    (dict(io_dtype=ws.GL_DTYPE_F32, flags=ws.GL_FLAG_OUT_F32), "mfma-f32"),
    (dict(io_dtype=ws.GL_DTYPE_F32), "mfma-f32"), (dict(io_dtype=ws.GL_DTYPE_F32, chunk=64), "mfma-f32"),
    (dict(io_dtype=ws.GL_DTYPE_F32, chunk=32), "generic-f32"),
    (dict(io_dtype=ws.GL_DTYPE_F32, d_in=100), "generic-f32"),
    (dict(io_dtype=ws.GL_DTYPE_F32, flags=ws.GL_FLAG_GENERIC), "generic-f32"),
    (dict(io_dtype=ws.GL_DTYPE_F64, d_in=32, d_out=32), "mfma-f64"),
    (dict(io_dtype=ws.GL_DTYPE_F64, d_in=32, d_out=20, chunk=64), "mfma-f64"),
    (dict(io_dtype=ws.GL_DTYPE_F64), "generic-f64"),
    (dict(io_dtype=ws.GL_DTYPE_F64, chunk=8), "generic-f64"),
    (dict(io_dtype=ws.GL_DTYPE_F64, chunk=16), "generic-f64"),
])
def test_chunk_and_flag_routing(kw, path):
    assert ws.path_name(desc(**kw)) == path


def test_null_desc():
    n = ctypes.c_size_t()
    assert ws.lib().gl_scan_saved_size(None, ctypes.byref(n)) == 1


def test_sizes_are_consistent():
    d = desc()
    s = ws.saved_size(d)
    f1, b1 = ws.workspace_size(d, True)
    f0, b0 = ws.workspace_size(d, False)
    assert s > 0 and b0 >= b1 + s - 256 and f0 == f1
    assert ws.path_name(d)


def test_segment_workspace():
    # one segment: the forward needs no workspace
    f, _ = ws.workspace_size(desc(T=4096, segments=1), True)
    assert f == 0
    # n segments: n fp32 states per sequence-head (+ their log-decays)
    f4, b4 = ws.workspace_size(desc(T=4096, segments=4), True)
    _, b1 = ws.workspace_size(desc(T=4096, segments=1), True)
    assert f4 >= 2 * 3 * 4 * 64 * 64 * 4 and b4 > b1
    # automatic: few heads and a long sequence are cut into segments, many
    # heads are not
    fa, _ = ws.workspace_size(desc(B=1, H=2, T=1 << 15), True)
    assert fa > 0
    fb, _ = ws.workspace_size(desc(B=8, H=16, T=4096), True)
    assert fb == 0
    # never more segments than chunks
    fc, _ = ws.workspace_size(desc(T=100, segments=50), True)
    assert fc == ws.workspace_size(desc(T=100, segments=2), True)[0]


FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _fwd(d, ptrs, ws_bytes=0):
    P = [ctypes.c_void_p(p) if p is not None else None for p in ptrs]
    return ws.lib().gl_scan_fwd(ctypes.byref(d), *P, ctypes.c_void_p(FAKE), ws_bytes, None)


def _bwd(d, ptrs, wsp, ws_bytes):
    P = [ctypes.c_void_p(p) if p is not None else None for p in ptrs]
    return ws.lib().gl_scan_bwd(ctypes.byref(d), *P, ctypes.c_void_p(wsp) if wsp else None,
                                ws_bytes, None)


def test_fwd_argument_errors_before_launch():
    d = desc()
    ok = [FAKE] * 6 + [None]  # x g eta alpha W0 y saved
    bad_null = list(ok)
    bad_null[2] = None
    assert _fwd(d, bad_null) == 1
    bad_al = list(ok)
    bad_al[0] = FAKE + 2
    assert _fwd(d, bad_al) == 3
    bad_saved = list(ok)
    bad_saved[6] = FAKE + 8
    assert _fwd(d, bad_saved) == 3
    assert b"aligned" in ws.lib().gl_last_error()


def test_fwd_segment_workspace_errors_before_launch():
    d = desc(T=4096, segments=4)
    need, _ = ws.workspace_size(d, True)
    P = [ctypes.c_void_p(FAKE)] * 6 + [None]
    L = ws.lib()
    assert L.gl_scan_fwd(ctypes.byref(d), *P, ctypes.c_void_p(FAKE), need - 1, None) == 4
    assert L.gl_scan_fwd(ctypes.byref(d), *P, None, need, None) == 1
    assert L.gl_scan_fwd(ctypes.byref(d), *P, ctypes.c_void_p(FAKE + 4), need, None) == 3


def test_bwd_argument_errors_before_launch():
    d = desc()
    ptrs = [FAKE] * 6 + [None] + [FAKE] * 5  # x g eta alpha W0 dy saved dx dg deta dalpha dW0
    _, need = ws.workspace_size(d, False)
    assert _bwd(d, ptrs, FAKE, need - 1) == 4
    assert _bwd(d, ptrs, None, need) == 1
    p2 = list(ptrs)
    p2[10] = None
    assert _bwd(d, p2, FAKE, need) == 1
    p3 = list(ptrs)
    p3[8] = FAKE + 4
    assert _bwd(d, p3, FAKE, need) == 3


def test_empty_forward_is_a_noop():
    # B*H*T == 0: nothing is launched and no pointer is needed
    for kw in (dict(T=0), dict(B=0), dict(H=0)):
        assert _fwd(desc(**kw), [None] * 7) == 0
    # an empty head count needs no dW0 either
    assert _bwd(desc(H=0), [None] * 12, None, 0) == 0


def _dec(fn, d, ptrs):
    P = [ctypes.c_void_p(p) if p is not None else None for p in ptrs]
    return getattr(ws.lib(), fn)(ctypes.byref(d) if d is not None else None, *P, None)


DEC_CALLS = (("gl_decode_readout", 4), ("gl_decode_update", 5), ("gl_decode_step", 8),
             ("gl_scan_final_state", 5), ("gl_costate_quadratic", 6))


def test_qkv_argument_errors_before_launch():
    L = ws.lib()
    P = lambda p: ctypes.c_void_p(p) if p is not None else None  # noqa: E731
    ok = [FAKE] * 6
    call = lambda d, ptrs, yp=FAKE: L.gl_scan_qkv_fwd(  # noqa: E731
        ctypes.byref(d), *[P(p) for p in ptrs], 0, P(yp), None)
    for i in range(6):
        p = list(ok)
        p[i] = None
        assert call(desc(), p) == 1
        p[i] = FAKE + 8
        assert call(desc(), p) == 3
    assert call(desc(), ok, None) == 1
    assert call(desc(d_in=129), ok) == 2
    assert call(desc(T=-1), ok) == 1
    assert call(desc(T=0), [None] * 6, None) == 0


def test_qkv_bwd_argument_errors_before_launch():
    L = ws.lib()
    P = lambda p: ctypes.c_void_p(p) if p is not None else None  # noqa: E731
    d = desc()
    n = ctypes.c_size_t()
    assert L.gl_scan_qkv_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    need = n.value
    assert need > 0
    assert L.gl_scan_qkv_workspace_size(ctypes.byref(desc(d_in=129)), ctypes.byref(n)) == 2
    assert L.gl_scan_qkv_workspace_size(ctypes.byref(d), None) == 1
    ok = [FAKE] * 13   # q k v eta alpha W0 dy dq dk dv deta dalpha dW0

    def call(dd, ptrs, wsp=FAKE, nb=need):
        pre, post = ptrs[:6], ptrs[6:]
        return L.gl_scan_qkv_bwd(ctypes.byref(dd), *[P(x) for x in pre], 0,
                                 *[P(x) for x in post], P(wsp), nb, None)
    for i in range(13):
        pp = list(ok)
        pp[i] = None
        assert call(d, pp) == 1, i
        pp[i] = FAKE + 8
        assert call(d, pp) == 3, i
    assert call(d, ok, nb=need - 1) == 4
    assert call(d, ok, wsp=None) == 1
    # empty: only dW0 is written (the zero sum), H == 0 needs nothing
    assert call(desc(H=0), [None] * 13, wsp=None, nb=0) == 0
    assert call(desc(T=0), [None] * 12 + [None], wsp=None, nb=0) == 1


@pytest.mark.parametrize("fn,nptr", DEC_CALLS)
def test_decode_argument_errors_before_launch(fn, nptr):
    ok = [FAKE] * nptr
    assert _dec(fn, None, ok) == 1
    for kw, code in ((dict(B=-1), 1), (dict(d_in=0), 1), (dict(io_dtype=5), 1),
                     (dict(d_out=129), 2), (dict(d_in=200), 2)):
        assert _dec(fn, desc(**kw), ok) == code, kw
    for i in range(nptr):
        p = list(ok)
        p[i] = None
        assert _dec(fn, desc(), p) == 1
        p[i] = FAKE + 4
        assert _dec(fn, desc(), p) == 3
    # no sequence-heads: nothing is launched and no pointer is needed
    assert _dec(fn, desc(B=0), [None] * nptr) == 0
    assert _dec(fn, desc(H=0), [None] * nptr) == 0


def test_decode_ignores_the_scan_only_fields():
    # chunk / segments / T have no meaning for one token; only the final state
    # checks T
    bad_scan = desc(chunk=48, segments=7, T=-3)
    assert _dec("gl_decode_readout", bad_scan, [None] * 4) == 1  # still needs pointers
    assert _dec("gl_scan_final_state", bad_scan, [FAKE] * 5) == 1  # negative T


def test_static_backward_refuses_a_workspace_beyond_its_scratch():
    # checked before the scratch address is taken or anything is launched
    d = desc(B=8, H=16, T=32768, d_in=128, d_out=128)
    _, need = ws.workspace_size(d, False)
    assert need > 64 << 20
    f = ctypes.c_void_p(FAKE)
    st = ws.lib().gl_scan_bwd_static(ctypes.byref(d), *([f] * 6), None, *([f] * 5), None)
    assert st == 4 and b"static scratch" in ws.lib().gl_last_error()
    # argument errors come first, as in gl_scan_bwd
    assert ws.lib().gl_scan_bwd_static(None, *([f] * 12), None) == 1


def test_qkv_forward_workspace():
    # bf16 at dk = dv = 128: the state entering every group of eight 64-token
    # chunks (bf16) in the caller's workspace; GL_FLAG_GENERIC and other
    # shapes need none; a workspace below the figure is refused before any
    # launch (fake device pointers)
    d = ws.make_desc(2, 3, 300, 128, 128, ws.GL_DTYPE_BF16)
    n = ctypes.c_size_t()
    assert ws.lib().gl_scan_qkv_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value >= 2 * 3 * 1 * 128 * 128 * 2
    dl = ws.make_desc(2, 3, 4096, 128, 128, ws.GL_DTYPE_BF16)
    nl = ctypes.c_size_t()
    assert ws.lib().gl_scan_qkv_fwd_workspace_size(ctypes.byref(dl), ctypes.byref(nl)) == 0
    assert nl.value >= 2 * 3 * 8 * 128 * 128 * 2
    for dd in (ws.make_desc(2, 3, 300, 128, 128, ws.GL_DTYPE_BF16, flags=ws.GL_FLAG_GENERIC),
               ws.make_desc(2, 3, 300, 64, 64, ws.GL_DTYPE_BF16),
               ws.make_desc(2, 3, 300, 128, 128, ws.GL_DTYPE_F32)):
        m = ctypes.c_size_t(1)
        assert ws.lib().gl_scan_qkv_fwd_workspace_size(ctypes.byref(dd), ctypes.byref(m)) == 0
        assert m.value == 0
    fake = ctypes.c_void_p(0x10000)
    st = ws.lib().gl_scan_qkv_fwd_ws(ctypes.byref(d), *([fake] * 6), 0, fake, fake, n.value - 256,
                                    None)
    assert st == 4
