"""The no-allocation backward (gl_scan_bwd_static, static scratch) against
gl_scan_bwd with a caller workspace: the same kernels on the same inputs, so
the results agree bit for bit; two calls in a row, the second smaller (the
scratch keeps the first call's contents), and a descriptor whose backward
needs more scratch than the static buffer holds is refused before launch."""
import ctypes

import pytest
import torch

import weight_scans_amd as ws
from parity_util import NAMES, to_device
from weight_scans_amd.synth import Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _pair(w, flags=0):
    inp = make_inputs(w)
    dev = to_device(inp, w.dtype)
    y, saved = ws.gl_scan_fwd(dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"],
                              flags=flags)
    ref = ws.gl_scan_bwd(dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"], dev["dy"],
                         saved, flags=flags)
    got = ws.gl_scan_bwd_static(dev["x"], dev["g"], dev["eta"], dev["alpha"], dev["W0"],
                                dev["dy"], saved, flags=flags)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    (Workload("na1", 4, 8, 2048, 64, 64, "bf16", "base", "gauss", 3001),
     Workload("na2", 2, 4, 513, 64, 64, "bf16", "mix", "gauss", 3002)),
    (Workload("na3", 2, 4, 4096, 128, 128, "bf16", "near1", "gauss", 3003),
     Workload("na4", 1, 2, 700, 128, 128, "bf16", "mix", "unit", 3004)),
    (Workload("na5", 2, 3, 300, 48, 40, "f64", "mix", "gauss", 3005),
     Workload("na6", 1, 2, 70, 20, 24, "f64", "base", "gauss", 3006)),
    # the fp32 matrix-core kernels (their adjoint and decay buffers in the scratch)
    (Workload("na7", 4, 8, 1024, 64, 64, "f32", "base", "gauss", 3007),
     Workload("na8", 1, 3, 130, 30, 50, "f32", "mix", "gauss", 3008)),
])
def test_static_scratch_matches_workspace(first, second):
    for w in (first, second):
        say(f"case {w}")
        ref, got = _pair(w)
        for n, a, b in zip(NAMES[1:], ref, got):
            assert torch.equal(a, b), (w.name, n)


def test_too_large_is_refused():
    # a long sequence without saved states: the recompute alone needs more
    # than the static scratch; nothing is launched
    d = ws.make_desc(8, 16, 32768, 128, 128, ws.GL_DTYPE_BF16)
    _, need = ws.workspace_size(d, False)
    assert need > 64 << 20
    fake = ctypes.c_void_p(0x10000)
    st = ws.lib().gl_scan_bwd_static(ctypes.byref(d), *([fake] * 6), None, *([fake] * 5), None)
    assert st == 4
    assert b"static scratch" in ws.lib().gl_last_error()
