"""Python entry points over the C ABI (argument marshalling only).

Every function takes CUDA (HIP) tensors, checks dtype/shape/contiguity,
passes raw device pointers and torch's current stream to ``libmhc.so`` and
returns the output tensors.  All arithmetic runs in the gfx950 kernels.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import LayerArgs, ProjOpts, check, lib

SOLVERS = {"newton": 0, "sinkhorn": 1}


def make_opts(solver="newton", max_iters=None, tol=None, warm_sweeps=None) -> ProjOpts:
    o = ProjOpts()
    check(lib().mhc_proj_opts_default(ctypes.byref(o)))
    if solver not in SOLVERS:
        raise ValueError(f"solver must be one of {sorted(SOLVERS)}")
    o.solver = SOLVERS[solver]
    if solver == "sinkhorn":
        o.max_iters = 1000
    if max_iters is not None:
        o.max_iters = int(max_iters)
    if tol is not None:
        o.tol = float(tol)
    if warm_sweeps is not None:
        o.warm_sweeps = int(warm_sweeps)
    return o


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, last_dims=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if last_dims is not None and tuple(t.shape[-len(last_dims):]) != tuple(last_dims):
        raise ValueError(f"{name} must have trailing shape {last_dims}, got {tuple(t.shape)}")


def birkhoff_fwd(logits: torch.Tensor, *, solver="newton", max_iters=None, tol=None,
                 warm_sweeps=None, out=None, return_iters=False):
    """Project [..., 4, 4] fp32 logits onto the doubly stochastic matrices.
    Returns P (and the uint8 iteration codes if ``return_iters``)."""
    _need(logits, "logits", torch.float32, (4, 4))
    B = logits.numel() // 16
    P = torch.empty_like(logits) if out is None else out
    if out is not None:
        _need(out, "out", torch.float32, (4, 4))
        if out.shape != logits.shape or out.device != logits.device:
            raise ValueError("out must match logits in shape and device")
    iters = torch.empty(logits.shape[:-2], dtype=torch.uint8, device=logits.device) if return_iters else None
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    with torch.cuda.device(logits.device):
        check(lib().mhc_birkhoff_fwd(_ptr(logits), _ptr(P), B, ctypes.byref(o), _ptr(iters),
                                     _stream(logits.device)))
    return (P, iters) if return_iters else P


def birkhoff_bwd(P: torch.Tensor, grad_P: torch.Tensor, out=None):
    """dL/dlogits from P = projection(logits) and dL/dP (fp32 [..., 4, 4])."""
    _need(P, "P", torch.float32, (4, 4))
    _need(grad_P, "grad_P", torch.float32, (4, 4))
    if P.shape != grad_P.shape or P.device != grad_P.device:
        raise ValueError("P and grad_P must match in shape and device")
    dA = torch.empty_like(P) if out is None else out
    if out is not None:
        _need(out, "out", torch.float32, (4, 4))
    with torch.cuda.device(P.device):
        check(lib().mhc_birkhoff_bwd(_ptr(P), _ptr(grad_P), _ptr(dA), P.numel() // 16,
                                     _stream(P.device)))
    return dA


def birkhoff_fwd_n(logits: torch.Tensor, *, solver="newton", max_iters=None, tol=None,
                   warm_sweeps=None, out=None, return_iters=False):
    """Project [..., n, n] fp32 logits (1 <= n <= 8) onto the doubly
    stochastic matrices (n = 4 runs the 4x4 kernels)."""
    if logits.dim() < 2 or logits.shape[-1] != logits.shape[-2]:
        raise ValueError("logits must be [..., n, n]")
    n = logits.shape[-1]
    _need(logits, "logits", torch.float32, (n, n))
    B = logits.numel() // (n * n)
    P = torch.empty_like(logits) if out is None else out
    if out is not None:
        _need(out, "out", torch.float32, (n, n))
        if out.shape != logits.shape or out.device != logits.device:
            raise ValueError("out must match logits in shape and device")
    iters = torch.empty(logits.shape[:-2], dtype=torch.uint8, device=logits.device) if return_iters else None
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    with torch.cuda.device(logits.device):
        check(lib().mhc_birkhoff_fwd_n(_ptr(logits), _ptr(P), B, n, ctypes.byref(o), _ptr(iters),
                                       _stream(logits.device)))
    return (P, iters) if return_iters else P


def birkhoff_bwd_n(P: torch.Tensor, grad_P: torch.Tensor, out=None):
    """dL/dlogits for [..., n, n] P = projection(logits) and dL/dP."""
    if P.dim() < 2 or P.shape[-1] != P.shape[-2]:
        raise ValueError("P must be [..., n, n]")
    n = P.shape[-1]
    _need(P, "P", torch.float32, (n, n))
    _need(grad_P, "grad_P", torch.float32, (n, n))
    if P.shape != grad_P.shape or P.device != grad_P.device:
        raise ValueError("P and grad_P must match in shape and device")
    dA = torch.empty_like(P) if out is None else out
    if out is not None:
        _need(out, "out", torch.float32, (n, n))
    with torch.cuda.device(P.device):
        check(lib().mhc_birkhoff_bwd_n(_ptr(P), _ptr(grad_P), _ptr(dA), P.numel() // (n * n), n,
                                       _stream(P.device)))
    return dA


def birkhoff_bwd_recompute(logits: torch.Tensor, grad_P: torch.Tensor, *, solver="newton",
                           max_iters=None, tol=None, warm_sweeps=None, out=None):
    """dL/dlogits from the logits and dL/dP: the projection is solved again in
    registers (same solver and options as the forward) and differentiated
    there, so P need not be kept between forward and backward."""
    _need(logits, "logits", torch.float32, (4, 4))
    _need(grad_P, "grad_P", torch.float32, (4, 4))
    if logits.shape != grad_P.shape or logits.device != grad_P.device:
        raise ValueError("logits and grad_P must match in shape and device")
    dA = torch.empty_like(logits) if out is None else out
    if out is not None:
        _need(out, "out", torch.float32, (4, 4))
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    with torch.cuda.device(logits.device):
        check(lib().mhc_birkhoff_bwd_recompute(_ptr(logits), _ptr(grad_P), _ptr(dA),
                                               logits.numel() // 16, ctypes.byref(o),
                                               _stream(logits.device)))
    return dA


def birkhoff_fwd_bwd(logits: torch.Tensor, grad_P: torch.Tensor, *, solver="newton",
                     max_iters=None, tol=None, warm_sweeps=None, out_P=None, out_grad=None,
                     return_iters=False):
    """P and dL/dlogits in one pass, for when dL/dP is known when the
    projection is computed (otherwise use birkhoff_fwd, then birkhoff_bwd).
    out_P may be ``logits`` itself and out_grad ``grad_P`` itself."""
    _need(logits, "logits", torch.float32, (4, 4))
    _need(grad_P, "grad_P", torch.float32, (4, 4))
    if logits.shape != grad_P.shape or logits.device != grad_P.device:
        raise ValueError("logits and grad_P must match in shape and device")
    P = torch.empty_like(logits) if out_P is None else out_P
    dA = torch.empty_like(logits) if out_grad is None else out_grad
    for t, name in ((P, "out_P"), (dA, "out_grad")):
        _need(t, name, torch.float32, (4, 4))
        if t.shape != logits.shape:
            raise ValueError(f"{name} must have the shape of logits")
    B = logits.numel() // 16
    it = torch.empty(logits.shape[:-2], dtype=torch.uint8, device=logits.device) if return_iters else None
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    with torch.cuda.device(logits.device):
        check(lib().mhc_birkhoff_fwd_bwd(_ptr(logits), _ptr(grad_P), _ptr(P), _ptr(dA), B,
                                         ctypes.byref(o), _ptr(it),
                                         _stream(logits.device)))
    return (P, dA, it) if return_iters else (P, dA)


class BirkhoffProjection(torch.autograd.Function):
    """Autograd wrapper.  By default it saves only P for the backward (nothing
    else from the forward solve is needed); with ``recompute`` it saves the
    logits instead and the backward solves the projection again."""

    @staticmethod
    def forward(ctx, logits, solver="newton", max_iters=None, tol=None, warm_sweeps=None,
                recompute=False):
        logits = logits.contiguous()
        P = birkhoff_fwd(logits, solver=solver, max_iters=max_iters, tol=tol,
                         warm_sweeps=warm_sweeps)
        ctx.recompute = recompute
        ctx.opts = (solver, max_iters, tol, warm_sweeps)
        ctx.save_for_backward(logits if recompute else P)
        return P

    @staticmethod
    def backward(ctx, grad_P):
        (saved,) = ctx.saved_tensors
        if ctx.recompute:
            solver, max_iters, tol, warm_sweeps = ctx.opts
            dA = birkhoff_bwd_recompute(saved, grad_P.contiguous(), solver=solver,
                                        max_iters=max_iters, tol=tol, warm_sweeps=warm_sweeps)
        else:
            dA = birkhoff_bwd(saved, grad_P.contiguous())
        return dA, None, None, None, None, None


def birkhoff_project(logits, **kw):
    """Differentiable projection (see BirkhoffProjection)."""
    return BirkhoffProjection.apply(logits, kw.get("solver", "newton"), kw.get("max_iters"),
                                    kw.get("tol"), kw.get("warm_sweeps"),
                                    bool(kw.get("recompute", False)))


def stream_mix(x: torch.Tensor, H: torch.Tensor = None, *, logits: torch.Tensor = None,
               out=None, return_H=False, solver="newton", max_iters=None, tol=None,
               warm_sweeps=None):
    """out[t,i,:] = sum_j H[t,i,j] x[t,j,:] for x [T,4,C] bf16.

    Pass either ``H`` [T,4,4] fp32, or ``logits`` [T,4,4] fp32 to project in
    the same kernel (then ``return_H`` also returns the projected H)."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 3:
        raise ValueError("x must be [T, n, C]")
    T, n, C = x.shape
    if (H is None) == (logits is None):
        raise ValueError("pass exactly one of H or logits")
    src = H if H is not None else logits
    _need(src, "H" if H is not None else "logits", torch.float32, (n, n))
    if src.shape[0] != T:
        raise ValueError("H/logits must have T rows")
    y = torch.empty_like(x) if out is None else out
    H_out = None
    if logits is not None and return_H:
        H_out = torch.empty_like(logits)
    o = make_opts(solver, max_iters, tol, warm_sweeps) if logits is not None else None
    with torch.cuda.device(x.device):
        check(lib().mhc_stream_mix(_ptr(x), _ptr(src), _ptr(H_out), _ptr(y), T, n, C,
                                   ctypes.byref(o) if o is not None else None,
                                   _stream(x.device)))
    return (y, H_out) if return_H else y


def stream_mix_bwd(x: torch.Tensor, H: torch.Tensor, grad_out: torch.Tensor, out=None):
    """(grad_x bf16 [T,4,C], grad_H fp32 [T,4,4]) of the stream mix; ``out``
    may be a preallocated (grad_x, grad_H) pair."""
    _need(x, "x", torch.bfloat16)
    _need(grad_out, "grad_out", torch.bfloat16)
    T, n, C = x.shape
    _need(H, "H", torch.float32, (n, n))
    if out is None:
        gx, gH = torch.empty_like(x), torch.empty_like(H)
    else:
        gx, gH = out
        _need(gx, "grad_x", torch.bfloat16)
        _need(gH, "grad_H", torch.float32, (n, n))
        if gx.shape != x.shape or gH.shape != H.shape:
            raise ValueError("out must be (grad_x like x, grad_H like H)")
    with torch.cuda.device(x.device):
        check(lib().mhc_stream_mix_bwd(_ptr(x), _ptr(H), _ptr(grad_out), _ptr(gx), _ptr(gH), T,
                                       n, C, _stream(x.device)))
    return gx, gH


N_MAPS = 24  # n*n + 2n for n = 4


def _layer_args(x, W, f, eps, opts):
    _need(x, "x", torch.bfloat16)
    if x.dim() != 3:
        raise ValueError("x must be [T, n, C]")
    T, n, C = x.shape
    _need(W, "W", torch.bfloat16)
    _need(f, "f", torch.bfloat16)
    if tuple(W.shape) != (n * n + 2 * n, n * C) or tuple(f.shape) != (T, C):
        raise ValueError("W must be [n*n+2n, n*C] and f [T, C]")
    a = LayerArgs()
    a.T, a.n, a.C, a.eps = T, n, C, float(eps)
    a.proj = ctypes.pointer(opts) if opts is not None else None
    a.x, a.W, a.f = x.data_ptr(), W.data_ptr(), f.data_ptr()
    return a


def layer_fwd(x, W, f, *, eps=1e-6, solver="newton", max_iters=None, tol=None,
              warm_sweeps=None):
    """Forward of one mHC layer step.  x [T,4,C], W [24,4C], f [T,C] bf16.
    Returns dict(u, x_out, rms, logits, H_pre, H_post, H_res)."""
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    a = _layer_args(x, W, f, eps, o)
    T, n, C = x.shape
    dev = x.device
    out = dict(u=torch.empty((T, C), dtype=torch.bfloat16, device=dev),
               x_out=torch.empty_like(x),
               rms=torch.empty(T, dtype=torch.float32, device=dev),
               logits=torch.empty((T, N_MAPS), dtype=torch.float32, device=dev),
               H_pre=torch.empty((T, n), dtype=torch.float32, device=dev),
               H_post=torch.empty((T, n), dtype=torch.float32, device=dev),
               H_res=torch.empty((T, n, n), dtype=torch.float32, device=dev))
    for k in ("u", "x_out", "rms", "logits", "H_pre", "H_post", "H_res"):
        setattr(a, k, out[k].data_ptr())
    with torch.cuda.device(dev):
        check(lib().mhc_layer_fwd(ctypes.byref(a), _stream(dev)))
    return out


def layer_fwd_into(x, W, f, out, *, eps=1e-6, solver="newton"):
    """layer_fwd writing into the tensors of a previous result dict ``out``."""
    o = make_opts(solver)
    a = _layer_args(x, W, f, eps, o)
    for k in ("u", "x_out", "rms", "logits", "H_pre", "H_post", "H_res"):
        setattr(a, k, out[k].data_ptr())
    with torch.cuda.device(x.device):
        check(lib().mhc_layer_fwd(ctypes.byref(a), _stream(x.device)))
    return out


def stream_mix_into(x, logits, H_out, out, solver="newton"):
    """Fused projection + stream mix into preallocated H_out and out."""
    T, n, C = x.shape
    o = make_opts(solver)
    with torch.cuda.device(x.device):
        check(lib().mhc_stream_mix(_ptr(x), _ptr(logits), _ptr(H_out), _ptr(out), T, n, C,
                                   ctypes.byref(o), _stream(x.device)))
    return out


def layer_workspace(T, C, device, n=4):
    nbytes = lib().mhc_layer_workspace_bytes(T, n, C)
    if nbytes < 0:
        raise ValueError("invalid layer shape")
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def layer_bwd(x, W, f, fwd, grad_x_out, grad_u, *, workspace=None, out=None):
    """Backward of one mHC layer step given the forward's outputs ``fwd``.
    Returns dict(grad_x, grad_f, grad_W, grad_logits)."""
    a = _layer_args(x, W, f, 1e-6, None)
    T, n, C = x.shape
    dev = x.device
    _need(grad_x_out, "grad_x_out", torch.bfloat16)
    _need(grad_u, "grad_u", torch.bfloat16)
    for k in ("rms", "logits", "H_pre", "H_post", "H_res"):
        _need(fwd[k], k, torch.float32)
        setattr(a, k, fwd[k].data_ptr())
    a.grad_x_out, a.grad_u = grad_x_out.data_ptr(), grad_u.data_ptr()
    if out is None:
        out = dict(grad_x=torch.empty_like(x), grad_f=torch.empty_like(f),
                   grad_W=torch.empty(W.shape, dtype=torch.float32, device=dev),
                   grad_logits=torch.empty((T, N_MAPS), dtype=torch.float32, device=dev))
    for k in ("grad_x", "grad_f", "grad_W", "grad_logits"):
        setattr(a, k, out[k].data_ptr())
    ws = layer_workspace(T, C, dev, n) if workspace is None else workspace
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    with torch.cuda.device(dev):
        check(lib().mhc_layer_bwd(ctypes.byref(a), _stream(dev)))
    return out
