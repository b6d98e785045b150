"""The Python binding refuses output buffers that do not fit, before anything
is enqueued.

Every caller-provided output is checked for dtype, contiguity, exact shape and
device.  Each case passes a short view into a larger buffer filled with a
sentinel: had the call gone through, the kernel would have written the whole
batch, past the view's end.  The test checks that ValueError (or TypeError for
a host tensor) is raised and that the buffer still holds only the sentinel.
"""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

SENT = 7.0


def _sentinel(shape, dtype=torch.float32):
    return torch.full(shape, SENT, dtype=dtype, device="cuda")


def _untouched(buf):
    torch.cuda.synchronize()
    assert bool((buf.float() == SENT).all()), "a refused call wrote to its buffer"


def test_projection_outputs_checked(gpu_lib):
    bp = gpu_lib
    B = 300
    A = torch.from_numpy(W.logits_batch("normal10", B, 7)).cuda()
    G = torch.from_numpy(W.grad_batch(B, 8)).cuda()
    P = bp.birkhoff_fwd(A)
    buf = _sentinel((B + 8, 4, 4))
    short = buf[:B - 1]
    for call in (lambda: bp.birkhoff_fwd(A, out=short),
                 lambda: bp.birkhoff_bwd(P, G, out=short),
                 lambda: bp.birkhoff_bwd_recompute(A, G, out=short),
                 lambda: bp.birkhoff_fwd_bwd(A, G, out_P=short),
                 lambda: bp.birkhoff_fwd_bwd(A, G, out_grad=short),
                 lambda: bp.birkhoff_fwd_n(A, out=short),
                 lambda: bp.birkhoff_bwd_n(P, G, out=short)):
        with pytest.raises(ValueError):
            call()
    # a mismatched gradient is refused too
    with pytest.raises(ValueError):
        bp.birkhoff_bwd(P, G[:B - 1])
    # n x n: 3x3 records, out one matrix short
    A3 = torch.from_numpy(W.logits_batch("normal10", B, 9, n=3)).cuda()
    P3 = bp.birkhoff_fwd_n(A3)
    buf3 = _sentinel((B + 8, 3, 3))
    with pytest.raises(ValueError):
        bp.birkhoff_fwd_n(A3, out=buf3[:B - 1])
    with pytest.raises(ValueError):
        bp.birkhoff_bwd_n(P3, P3, out=buf3[:B - 1])
    # a host tensor as output
    with pytest.raises(TypeError):
        bp.birkhoff_fwd(A, out=torch.empty(B, 4, 4))
    _untouched(buf)
    _untouched(buf3)


def test_mix_outputs_checked(gpu_lib):
    bp = gpu_lib
    T, C = 40, 64
    x, logits = W.mix_inputs(T, C, seed=21, device=torch.device("cuda"))
    H = bp.birkhoff_fwd(logits)
    ybuf = _sentinel((T + 4, 4, C), torch.bfloat16)
    hbuf = _sentinel((T + 4, 4, 4))
    with pytest.raises(ValueError):
        bp.stream_mix(x, H, out=ybuf[:T - 1])
    with pytest.raises(ValueError):
        bp.stream_mix(x, logits=logits, out=ybuf[:T], return_H=True, H_out=hbuf[:T - 1])
    with pytest.raises(ValueError):
        bp.ops.stream_mix_into(x, logits, hbuf[:T], ybuf[:T - 1])
    with pytest.raises(ValueError):
        bp.stream_mix(x, H[:T - 1])
    g = torch.randn(T, 4, C, device="cuda").to(torch.bfloat16)
    with pytest.raises(ValueError):
        bp.stream_mix_bwd(x, H, g, out=(ybuf[:T - 1], hbuf[:T]))
    with pytest.raises(ValueError):
        bp.stream_mix_bwd(x, H, g, out=(ybuf[:T], hbuf[:T - 1]))
    _untouched(ybuf)
    _untouched(hbuf)


def test_layer_outputs_checked(gpu_lib):
    bp = gpu_lib
    T, C = 70, 64
    inp = W.layer_inputs(T, C, seed=22)
    x, Wt, f, dxo, du = inp["x"], inp["W"], inp["f"], inp["dx_out"], inp["du"]
    fw = bp.layer_fwd(x, Wt, f)
    ok = bp.layer_bwd(x, Wt, f, fw, dxo, du)
    torch.cuda.synchronize()
    wbuf = _sentinel((24 + 2, 4 * C))
    bad = dict(ok)
    bad["grad_W"] = wbuf[:23]
    with pytest.raises(ValueError):
        bp.layer_bwd(x, Wt, f, fw, dxo, du, out=bad)
    lbuf = _sentinel((T + 4, 24))
    bad = dict(ok)
    bad["grad_logits"] = lbuf[:T - 1]
    with pytest.raises(ValueError):
        bp.layer_bwd(x, Wt, f, fw, dxo, du, out=bad)
    # forward state of the wrong length
    short_fw = dict(fw)
    short_fw["H_res"] = fw["H_res"][:T - 1]
    with pytest.raises(ValueError):
        bp.layer_bwd(x, Wt, f, short_fw, dxo, du)
    with pytest.raises(ValueError):
        bp.layer_bwd(x, Wt, f, fw, dxo[:T - 1], du)
    fbuf = _sentinel((T + 4, C), torch.bfloat16)
    bad_fw = dict(fw)
    bad_fw["u"] = fbuf[:T - 1]
    with pytest.raises(ValueError):
        bp.layer_fwd(x, Wt, f, out=bad_fw)
    # a workspace of the wrong dtype
    with pytest.raises(TypeError):
        bp.layer_bwd(x, Wt, f, fw, dxo, du, workspace=torch.empty(16, device="cuda"))
    _untouched(wbuf)
    _untouched(lbuf)
    _untouched(fbuf)
