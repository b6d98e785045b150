"""mhc_layer_bwd_noalloc against mhc_layer_bwd.

The allocation-free backward runs the same kernels with the library's own
device scratch as the workspace, so its outputs must equal those of the
backward with a caller-provided workspace bit for bit.  Three calls in a row,
each smaller than the one before (the scratch keeps the previous call's
contents), every output pre-filled with NaN so that anything not written
shows.  The first shape is the largest the 64 MiB scratch is sized for in
practice (C = 7168, the workload's width).
"""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(16384, 7168), (2048 + 37, 512), (300, 256)]


def _nan_out(T, n, C, dev):
    nan = float("nan")
    return dict(grad_x=torch.full((T, n, C), nan, dtype=torch.bfloat16, device=dev),
                grad_f=torch.full((T, C), nan, dtype=torch.bfloat16, device=dev),
                grad_W=torch.full((24, n * C), nan, dtype=torch.float32, device=dev),
                grad_logits=torch.full((T, 24), nan, dtype=torch.float32, device=dev))


def test_noalloc_matches_workspace_backward(gpu_lib):
    bp = gpu_lib
    lib = bp.lib()
    for i, (T, C) in enumerate(SHAPES):
        print(f"noalloc call {i}: T={T} C={C}", flush=True)
        need = lib.mhc_layer_workspace_bytes(T, 4, C)
        assert 0 < need <= 64 << 20
        inp = W.layer_inputs(T, C, seed=60 + i)
        x, Wt, f, dxo, du = inp["x"], inp["W"], inp["f"], inp["dx_out"], inp["du"]
        fw = bp.layer_fwd(x, Wt, f)
        ref = bp.layer_bwd(x, Wt, f, fw, dxo, du)
        got = bp.layer_bwd_noalloc(x, Wt, f, fw, dxo, du, out=_nan_out(T, 4, C, x.device))
        torch.cuda.synchronize()
        for k in ("grad_x", "grad_f", "grad_W", "grad_logits"):
            assert torch.equal(got[k], ref[k]), f"call {i} T={T} C={C}: {k} differs"
        del inp, x, Wt, f, dxo, du, fw, ref, got
        torch.cuda.empty_cache()


def test_noalloc_refuses_shapes_beyond_its_scratch(gpu_lib):
    """Refused on the host before anything is enqueued (fake, never
    dereferenced pointers: the size check comes first)."""
    import ctypes
    from birkhoff_projection_amd._lib import LayerArgs
    lib = gpu_lib.lib()
    a = LayerArgs()
    a.T, a.n, a.C, a.eps = 262144, 4, 7168, 1e-6
    assert lib.mhc_layer_workspace_bytes(a.T, 4, a.C) > 64 << 20
    for k, (name, _) in enumerate(LayerArgs._fields_[5:-2]):
        setattr(a, name, 0x10000 + (k + 1) * (1 << 34))
    assert lib.mhc_layer_bwd_noalloc(ctypes.byref(a), None) == 1
    assert b"scratch" in lib.mhc_last_error()
