"""Host-side checks of the C ABI: the library loads, exports every function
include/mhc.h declares, and rejects bad arguments before touching the GPU.
No GPU needed (only error paths and empty batches are called)."""
import ctypes
import os
import re

import pytest

from birkhoff_projection_amd import _lib
from birkhoff_projection_amd._lib import ProjOpts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

INVALID, UNSUPPORTED = 1, 2
FAKE = 0x10000  # aligned address that is never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "mhc_birkhoff_fwd" in names and "mhc_stream_mix" in names
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_abi_version_and_strings(L):
    assert L.mhc_abi_version() == 4
    assert L.mhc_status_string(0) == b"ok"
    assert L.mhc_status_string(1) == b"invalid argument"
    assert L.mhc_status_string(2) == b"unsupported"
    assert L.mhc_status_string(3) == b"kernel launch failed"


def test_default_opts(L):
    o = ProjOpts()
    assert L.mhc_proj_opts_default(ctypes.byref(o)) == 0
    # -1: the solver's own limits (30 Newton iterations, 1000 Sinkhorn sweeps)
    assert (o.solver, o.max_iters, o.warm_sweeps) == (0, -1, -1)
    assert abs(o.tol - 1e-6) < 1e-12
    assert L.mhc_proj_opts_default(None) == INVALID


def test_empty_batch_is_noop(L):
    assert L.mhc_birkhoff_fwd(None, None, 0, None, None, None) == 0
    assert L.mhc_birkhoff_bwd(None, None, None, 0, None) == 0
    assert L.mhc_birkhoff_bwd_recompute(None, None, None, 0, None, None) == 0
    assert L.mhc_stream_mix(None, None, None, None, 0, 4, 8, None, None) == 0
    assert L.mhc_stream_mix_bwd(None, None, None, None, None, 0, 4, 8, None) == 0


def _err(L):
    return L.mhc_last_error().decode()


def test_fwd_argument_errors(L):
    assert L.mhc_birkhoff_fwd(FAKE, FAKE, -1, None, None, None) == INVALID
    assert "out of range" in _err(L)
    assert L.mhc_birkhoff_fwd(None, FAKE, 5, None, None, None) == INVALID
    assert L.mhc_birkhoff_fwd(FAKE + 4, FAKE + 4096, 5, None, None, None) == INVALID
    assert "aligned" in _err(L)
    # partial overlap of P and logits
    assert L.mhc_birkhoff_fwd(FAKE, FAKE + 64, 5, None, None, None) == INVALID
    assert "overlap" in _err(L)
    for field, value in (("solver", 3), ("max_iters", 0), ("max_iters", -2), ("max_iters", 10001),
                         ("tol", -1.0), ("tol", float("nan")), ("warm_sweeps", 65),
                         ("warm_sweeps", -2)):
        o = ProjOpts()
        L.mhc_proj_opts_default(ctypes.byref(o))
        setattr(o, field, value)
        assert L.mhc_birkhoff_fwd(FAKE, FAKE, 5, ctypes.byref(o), None, None) == INVALID, field
        assert field in _err(L)


def test_bwd_argument_errors(L):
    assert L.mhc_birkhoff_bwd(FAKE, FAKE, FAKE, -3, None) == INVALID
    assert L.mhc_birkhoff_bwd(FAKE, None, FAKE, 3, None) == INVALID
    assert L.mhc_birkhoff_bwd(FAKE, FAKE + 8192, FAKE + 8, 3, None) == INVALID
    # grad_logits may not overlap P at all
    assert L.mhc_birkhoff_bwd(FAKE, FAKE + 8192, FAKE, 3, None) == INVALID
    assert "overlaps P" in _err(L)


def test_fwd_bwd_argument_errors(L):
    """mhc_birkhoff_fwd_bwd: B = 0 is a no-op; NULL, misalignment and every
    overlap other than P == logits and grad_logits == grad_P are rejected
    before anything is enqueued (FAKE pointers are never dereferenced)."""
    f = L.mhc_birkhoff_fwd_bwd
    A, G, P, D = FAKE, FAKE + 8192, FAKE + 16384, FAKE + 24576
    assert f(None, None, None, None, 0, None, None, None) == 0
    assert f(A, G, P, D, -1, None, None, None) == INVALID
    assert f(A, G, None, D, 3, None, None, None) == INVALID
    assert "NULL" in _err(L)
    assert f(A, G, P + 4, D, 3, None, None, None) == INVALID
    assert "aligned" in _err(L)
    assert f(A, G, A + 64, D, 3, None, None, None) == INVALID
    assert "P partially overlaps logits" in _err(L)
    assert f(A, G, P, G + 64, 3, None, None, None) == INVALID
    assert "grad_logits partially overlaps grad_P" in _err(L)
    assert f(A, G, G, D, 3, None, None, None) == INVALID
    assert "P overlaps grad_P or grad_logits" in _err(L)
    assert f(A, G, P, P, 3, None, None, None) == INVALID
    assert "P overlaps grad_P or grad_logits" in _err(L)
    assert f(A, G, P, A, 3, None, None, None) == INVALID
    assert "grad_logits overlaps logits" in _err(L)
    assert f(A, G, P, D, 3, None, ctypes.c_void_p(A + 16), None) == INVALID
    assert "iters overlaps" in _err(L)
    o = ProjOpts()
    L.mhc_proj_opts_default(ctypes.byref(o))
    o.warm_sweeps = -2
    assert f(A, G, P, D, 3, ctypes.byref(o), None, None) == INVALID
    assert "warm_sweeps" in _err(L)


def test_pipeline_step_argument_errors(L):
    """mhc_birkhoff_pipeline_step: both batches empty is a no-op; each half is
    checked as mhc_birkhoff_fwd / mhc_birkhoff_bwd check it, and across the
    halves every output is checked against every array of the other half
    (inputs of both may share memory).  FAKE pointers are never dereferenced:
    every call below fails validation."""
    f = L.mhc_birkhoff_pipeline_step
    A, P, Pb, G, D = FAKE, FAKE + 8192, FAKE + 16384, FAKE + 24576, FAKE + 32768
    assert f(None, None, 0, None, None, None, None, None, 0, None) == 0
    assert f(A, P, -1, None, None, Pb, G, D, 3, None) == INVALID
    assert "B=-1" in _err(L)
    assert f(A, P, 3, None, None, Pb, G, D, -1, None) == INVALID
    assert "B_bwd" in _err(L)
    # the forward half as mhc_birkhoff_fwd checks it
    assert f(A, None, 3, None, None, Pb, G, D, 3, None) == INVALID
    assert f(A, A + 64, 3, None, None, Pb, G, D, 3, None) == INVALID
    assert "P partially overlaps logits" in _err(L)
    # the backward half as mhc_birkhoff_bwd checks it
    assert f(A, P, 3, None, None, Pb, G, Pb, 3, None) == INVALID
    assert "grad_logits overlaps P" in _err(L)
    assert f(A, P, 3, None, None, Pb, G + 4, D, 3, None) == INVALID
    assert "aligned" in _err(L)
    # across the halves
    for Pf in (Pb, G + 64, D):
        assert f(A, Pf, 3, None, None, Pb, G, D, 3, None) == INVALID
        assert "P overlaps P_bwd, grad_P or grad_logits" in _err(L)
    assert f(A, P, 3, None, None, Pb, G, A + 64, 3, None) == INVALID
    assert "grad_logits overlaps logits" in _err(L)
    assert f(A, P, 3, None, None, Pb, G, P, 3, None) == INVALID  # both write P's memory
    assert "P overlaps P_bwd, grad_P or grad_logits" in _err(L)
    assert f(A, P, 3, None, ctypes.c_void_p(G + 8), Pb, G, D, 3, None) == INVALID
    assert "iters overlaps" in _err(L)
    # a bad half is refused even when the other one is empty
    assert f(A, A + 64, 3, None, None, None, None, None, 0, None) == INVALID
    assert f(None, None, 0, None, None, Pb, G, Pb, 3, None) == INVALID
    o = ProjOpts()
    L.mhc_proj_opts_default(ctypes.byref(o))
    o.max_iters = 0
    assert f(A, P, 3, ctypes.byref(o), None, Pb, G, D, 3, None) == INVALID
    assert "max_iters" in _err(L)


def test_bwd_recompute_argument_errors(L):
    assert L.mhc_birkhoff_bwd_recompute(None, None, None, 0, None, None) == 0
    assert L.mhc_birkhoff_bwd_recompute(FAKE, FAKE, FAKE, -1, None, None) == INVALID
    assert L.mhc_birkhoff_bwd_recompute(FAKE, None, FAKE, 3, None, None) == INVALID
    assert L.mhc_birkhoff_bwd_recompute(FAKE + 4, FAKE + 8192, FAKE + 16384, 3, None, None) == INVALID
    assert "aligned" in _err(L)
    # exact aliasing of either input is allowed, partial overlap is not
    assert L.mhc_birkhoff_bwd_recompute(FAKE, FAKE + 8192, FAKE + 64, 3, None, None) == INVALID
    assert "overlaps logits" in _err(L)
    assert L.mhc_birkhoff_bwd_recompute(FAKE, FAKE + 8192, FAKE + 8192 + 64, 3, None, None) == INVALID
    assert "overlaps grad_P" in _err(L)
    o = ProjOpts()
    L.mhc_proj_opts_default(ctypes.byref(o))
    o.max_iters = 0
    assert L.mhc_birkhoff_bwd_recompute(FAKE, FAKE + 8192, FAKE + 16384, 3, ctypes.byref(o), None) == INVALID
    assert "max_iters" in _err(L)


def test_n_argument_errors(L):
    assert L.mhc_birkhoff_fwd_n(FAKE, FAKE, 5, 9, None, None, None) == UNSUPPORTED
    assert L.mhc_birkhoff_fwd_n(FAKE, FAKE, 5, 0, None, None, None) == UNSUPPORTED
    assert L.mhc_birkhoff_bwd_n(FAKE, FAKE, FAKE, 5, 9, None) == UNSUPPORTED
    assert L.mhc_birkhoff_fwd_n(None, None, 0, 3, None, None, None) == 0
    assert L.mhc_birkhoff_bwd_n(None, None, None, 0, 3, None) == 0
    assert L.mhc_birkhoff_fwd_n(FAKE + 2, FAKE + 4096, 5, 3, None, None, None) == INVALID
    assert "aligned" in _err(L)
    # 4-byte alignment suffices for n != 4; n = 4 keeps its 16-byte rule
    assert L.mhc_birkhoff_fwd_n(FAKE + 4, FAKE + 4, 5, 4, None, None, None) == INVALID
    assert "16-byte" in _err(L)
    assert L.mhc_birkhoff_fwd_n(FAKE, FAKE + 36, 5, 3, None, None, None) == INVALID
    assert "overlap" in _err(L)
    assert L.mhc_birkhoff_bwd_n(FAKE, FAKE + 8192, FAKE + 36, 5, 3, None) == INVALID
    assert "overlaps P" in _err(L)
    o = ProjOpts()
    L.mhc_proj_opts_default(ctypes.byref(o))
    o.solver = 5
    assert L.mhc_birkhoff_fwd_n(FAKE, FAKE, 5, 3, ctypes.byref(o), None, None) == INVALID


def test_mix_argument_errors(L):
    x, h, o = FAKE, FAKE + (1 << 24), FAKE + (1 << 25)
    assert L.mhc_stream_mix(x, h, None, o, 4, 3, 64, None, None) == UNSUPPORTED
    assert L.mhc_stream_mix(x, h, None, o, 4, 4, 12, None, None) == INVALID
    assert L.mhc_stream_mix(x, h, None, o, 4, 4, 0, None, None) == INVALID
    assert L.mhc_stream_mix(x, h, None, o, -1, 4, 64, None, None) == INVALID
    assert L.mhc_stream_mix(x, None, None, o, 4, 4, 64, None, None) == INVALID
    assert L.mhc_stream_mix(x + 2, h, None, o, 4, 4, 64, None, None) == INVALID
    # out overlapping x
    assert L.mhc_stream_mix(x, h, None, x + 256, 4, 4, 64, None, None) == INVALID
    bad = ProjOpts()
    L.mhc_proj_opts_default(ctypes.byref(bad))
    bad.solver = 7
    assert L.mhc_stream_mix(x, h, None, o, 4, 4, 64, ctypes.byref(bad), None) == INVALID
    assert L.mhc_stream_mix_bwd(x, h, o, FAKE + (1 << 26), FAKE + (1 << 27), 4, 5, 64, None) == UNSUPPORTED
    assert L.mhc_stream_mix_bwd(x, h, o, x, FAKE + (1 << 27), 4, 4, 64, None) == INVALID


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import birkhoff_projection_amd as bp
    with pytest.raises(TypeError):
        bp.birkhoff_fwd(torch.zeros(3, 4, 4))
    with pytest.raises(TypeError):
        bp.stream_mix(torch.zeros(3, 4, 8, dtype=torch.bfloat16), torch.zeros(3, 4, 4))


def test_layer_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of mhc_layer_args has the C layout (offsets checked
    with a C program compiled against include/mhc.h)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in _lib.LayerArgs._fields_]
    src = tmp_path / "off.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mhc.h"\nint main(void){\n'
                   + "".join(f'printf("%zu\\n", offsetof(mhc_layer_args, {f}));\n' for f in fields)
                   + 'printf("%zu\\n", sizeof(mhc_layer_args));\nprintf("%zu\\n", sizeof(mhc_proj_opts));\nreturn 0;}\n')
    exe = tmp_path / "off"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [getattr(_lib.LayerArgs, f).offset for f in fields] + [ctypes.sizeof(_lib.LayerArgs), ctypes.sizeof(ProjOpts)]
    assert got == want


def test_layer_argument_errors(L):
    a = _lib.LayerArgs()
    a.T, a.n, a.C, a.eps = 4, 4, 64, 1e-6
    names = ["x", "W", "f", "u", "x_out", "rms", "logits", "H_pre", "H_post", "H_res",
             "grad_x_out", "grad_u", "grad_x", "grad_f", "grad_W", "grad_logits", "workspace"]
    for i, nm in enumerate(names):
        setattr(a, nm, FAKE + (i + 1) * (1 << 24))
    a.workspace_bytes = L.mhc_layer_workspace_bytes(4, 4, 64)
    assert a.workspace_bytes > 0
    assert L.mhc_layer_workspace_bytes(4, 3, 64) == -1
    assert L.mhc_layer_workspace_bytes(4, 4, 96) == -1
    a.n = 3
    assert L.mhc_layer_fwd(ctypes.byref(a), None) == UNSUPPORTED
    a.n = 4
    a.C = 96
    assert L.mhc_layer_fwd(ctypes.byref(a), None) == INVALID
    a.C = 64
    a.eps = 0.0
    assert L.mhc_layer_fwd(ctypes.byref(a), None) == INVALID
    a.eps = 1e-6
    a.x = None
    assert L.mhc_layer_fwd(ctypes.byref(a), None) == INVALID
    assert "x must not be NULL" in _err(L)
    a.x = FAKE + (1 << 24)
    a.u = a.x  # output overlapping an input
    assert L.mhc_layer_fwd(ctypes.byref(a), None) == INVALID
    assert "overlaps" in _err(L)
    a.u = FAKE + 4 * (1 << 24)
    a.workspace_bytes -= 1
    assert L.mhc_layer_bwd(ctypes.byref(a), None) == INVALID
    assert "workspace" in _err(L)
    assert L.mhc_layer_fwd(None, None) == INVALID
    a.T = 0
    assert L.mhc_layer_fwd(ctypes.byref(a), None) == 0
    assert L.mhc_layer_bwd(ctypes.byref(a), None) == 0


def _header_int(name):
    m = re.search(r"#define\s+" + name + r"\s+\(\(int64_t\)(\d+)\)", open(HEADER).read())
    assert m, name
    return int(m.group(1))


def test_size_limits_at_the_boundary(L):
    """B and T one past MHC_MAX_BATCH / MHC_MAX_TOKENS are rejected as out of
    range before anything else is looked at; at the limit the check passes and
    the (misaligned) pointers are what fails.  The limits keep every launch
    below 2^32 work-items: 4 lanes per matrix in the 4x4 backward, 16 per
    token in the token kernels."""
    MB, MT = _header_int("MHC_MAX_BATCH"), _header_int("MHC_MAX_TOKENS")
    assert MB == (1 << 30) - 64 and 4 * MB < (1 << 32)
    assert MT == (1 << 28) - 16 and 16 * MT < (1 << 32)
    bad = FAKE + 2  # misaligned for every call (4x4: 16 bytes, n x n: 4): fails after the range check
    calls = [
        lambda b: L.mhc_birkhoff_fwd(bad, bad, b, None, None, None),
        lambda b: L.mhc_birkhoff_bwd(bad, bad, bad, b, None),
        lambda b: L.mhc_birkhoff_bwd_recompute(bad, bad, bad, b, None, None),
        lambda b: L.mhc_birkhoff_fwd_bwd(bad, bad, bad, bad, b, None, None, None),
        lambda b: L.mhc_birkhoff_fwd_n(bad, bad, b, 3, None, None, None),
        lambda b: L.mhc_birkhoff_bwd_n(bad, bad, bad, b, 3, None),
    ]
    for call in calls:
        assert call(MB + 1) == INVALID and "out of range" in _err(L)
        assert call(MB) == INVALID and "out of range" not in _err(L)
    tcalls = [
        lambda t: L.mhc_stream_mix(bad, bad, None, bad, t, 4, 64, None, None),
        lambda t: L.mhc_stream_mix_bwd(bad, bad, bad, bad, bad, t, 4, 64, None),
    ]
    for call in tcalls:
        assert call(MT + 1) == INVALID and "out of range" in _err(L)
        assert call(MT) == INVALID and "out of range" not in _err(L)
    assert L.mhc_layer_workspace_bytes(MT + 1, 4, 64) == -1
    assert L.mhc_layer_workspace_bytes(MT, 4, 64) > 0


def test_sinkhorn_default_sweeps_resolved_by_the_library(L):
    """max_iters = -1 (the default) with the Sinkhorn solver is accepted; an
    explicit count is range-checked whatever the solver."""
    o = ProjOpts()
    L.mhc_proj_opts_default(ctypes.byref(o))
    o.solver = 1
    # passes option validation, then fails on the NULL pointers
    assert L.mhc_birkhoff_fwd(None, FAKE, 5, ctypes.byref(o), None, None) == INVALID
    assert "NULL" in _err(L)
    o.max_iters = 10001
    assert L.mhc_birkhoff_fwd(None, FAKE, 5, ctypes.byref(o), None, None) == INVALID
    assert "max_iters" in _err(L)


def test_layer_bwd_noalloc_refuses_before_touching_the_device(L):
    """mhc_layer_bwd_noalloc checks the shape against its fixed scratch
    (MHC_LAYER_NOALLOC_SCRATCH_BYTES) and the pointers on the host, before it
    asks for a device (fake pointers, never dereferenced)."""
    m = re.search(r"#define\s+MHC_LAYER_NOALLOC_SCRATCH_BYTES\s+\(\(int64_t\)(\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) == 64 << 20
    a = _lib.LayerArgs()
    a.T, a.n, a.C, a.eps = 262144, 4, 7168, 1e-6
    assert L.mhc_layer_workspace_bytes(a.T, 4, a.C) > 64 << 20
    names = ["x", "W", "f", "u", "x_out", "rms", "logits", "H_pre", "H_post", "H_res",
             "grad_x_out", "grad_u", "grad_x", "grad_f", "grad_W", "grad_logits"]
    for i, nm in enumerate(names):
        setattr(a, nm, FAKE + (i + 1) * (1 << 36))
    assert L.mhc_layer_bwd_noalloc(ctypes.byref(a), None) == INVALID
    assert "scratch" in _err(L)
    a.T = 65536  # fits (49.6 MiB), but an output overlapping an input is refused
    assert 0 < L.mhc_layer_workspace_bytes(a.T, 4, a.C) <= 64 << 20
    a.grad_x = a.x
    assert L.mhc_layer_bwd_noalloc(ctypes.byref(a), None) == INVALID
    assert "overlaps" in _err(L)
    a.n = 3
    assert L.mhc_layer_bwd_noalloc(ctypes.byref(a), None) == UNSUPPORTED
    a.n, a.T = 4, 0
    assert L.mhc_layer_bwd_noalloc(ctypes.byref(a), None) == 0
    assert L.mhc_layer_bwd_noalloc(None, None) == INVALID
