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


def _same(t, name, like, like_name):
    """t (already checked by _need) has exactly like's shape and device."""
    if tuple(t.shape) != tuple(like.shape):
        raise ValueError(f"{name} must have the shape of {like_name} {tuple(like.shape)}, "
                         f"got {tuple(t.shape)}")
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}, got {t.device}")


def _out(out, name, dtype, shape, device):
    """A caller-provided output: a contiguous CUDA tensor of exactly ``shape``
    and ``dtype`` on ``device`` (a short or misplaced buffer would let the
    kernel write past its allocation), or a new one if ``out`` is None."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(out, name, dtype)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.device != device:
        raise ValueError(f"{name} must be on {device}, got {out.device}")
    return out


def birkhoff_fwd(logits: torch.Tensor, *, solver="newton", max_iters=None, tol=None,
                 warm_sweeps=None, out=None, return_iters=False):
    """Project [..., 4, 4] fp32 logits onto the doubly stochastic matrices.
    Returns P (and the uint8 iteration codes if ``return_iters``)."""
    _need(logits, "logits", torch.float32, (4, 4))
    B = logits.numel() // 16
    P = _out(out, "out", torch.float32, logits.shape, logits.device)
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
    _same(grad_P, "grad_P", P, "P")
    dA = _out(out, "out", torch.float32, P.shape, P.device)
    with torch.cuda.device(P.device):
        check(lib().mhc_birkhoff_bwd(_ptr(P), _ptr(grad_P), _ptr(dA), P.numel() // 16,
                                     _stream(P.device)))
    return dA


def birkhoff_pipeline_step(logits: torch.Tensor, P_bwd: torch.Tensor, grad_P: torch.Tensor, *,
                           solver="newton", max_iters=None, tol=None, warm_sweeps=None, out=None,
                           out_grad=None, return_iters=False):
    """The forward of one batch and the backward of another, independent one
    in a single launch: P = projection(logits) and dL/dlogits of the other
    batch from its P_bwd and dL/dP.  P is bit for bit birkhoff_fwd's; the
    gradient is birkhoff_bwd_recompute's arithmetic (bit for bit when P_bwd
    is the forward's P of those logits) and birkhoff_bwd's up to fp32
    rounding.  Both batches are [..., 4, 4] fp32 on one device, either may be
    empty, out may be logits and out_grad grad_P.  Returns (P, grad) (and the
    forward's iteration codes if ``return_iters``)."""
    _need(logits, "logits", torch.float32, (4, 4))
    _need(P_bwd, "P_bwd", torch.float32, (4, 4))
    _need(grad_P, "grad_P", torch.float32, (4, 4))
    _same(grad_P, "grad_P", P_bwd, "P_bwd")
    if P_bwd.device != logits.device:
        raise ValueError(f"P_bwd must be on {logits.device}, got {P_bwd.device}")
    P = _out(out, "out", torch.float32, logits.shape, logits.device)
    dA = _out(out_grad, "out_grad", torch.float32, P_bwd.shape, P_bwd.device)
    it = torch.empty(logits.shape[:-2], dtype=torch.uint8, device=logits.device) if return_iters else None
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    with torch.cuda.device(logits.device):
        check(lib().mhc_birkhoff_pipeline_step(_ptr(logits), _ptr(P), logits.numel() // 16,
                                               ctypes.byref(o), _ptr(it), _ptr(P_bwd),
                                               _ptr(grad_P), _ptr(dA), P_bwd.numel() // 16,
                                               _stream(logits.device)))
    return (P, dA, it) if return_iters else (P, dA)


def birkhoff_fwd_n(logits: torch.Tensor, *, solver="newton", max_iters=None, tol=None,
                   warm_sweeps=None, out=None, return_iters=False):
    """Project [..., n, n] fp32 logits (1 <= n <= 8) onto the doubly
    stochastic matrices (n = 4 runs the 4x4 kernels)."""
    if logits.dim() < 2 or logits.shape[-1] != logits.shape[-2]:
        raise ValueError("logits must be [..., n, n]")
    n = logits.shape[-1]
    _need(logits, "logits", torch.float32, (n, n))
    B = logits.numel() // (n * n)
    P = _out(out, "out", torch.float32, logits.shape, logits.device)
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
    _same(grad_P, "grad_P", P, "P")
    dA = _out(out, "out", torch.float32, P.shape, P.device)
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
    _same(grad_P, "grad_P", logits, "logits")
    dA = _out(out, "out", torch.float32, logits.shape, logits.device)
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
    _same(grad_P, "grad_P", logits, "logits")
    P = _out(out_P, "out_P", torch.float32, logits.shape, logits.device)
    dA = _out(out_grad, "out_grad", torch.float32, logits.shape, logits.device)
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
               out=None, return_H=False, H_out=None, solver="newton", max_iters=None, tol=None,
               warm_sweeps=None):
    """out[t,i,:] = sum_j H[t,i,j] x[t,j,:] for x [T,4,C] bf16.

    Pass either ``H`` [T,4,4] fp32, or ``logits`` [T,4,4] fp32 to project in
    the same kernel (then ``return_H`` also returns the projected H, written
    into ``H_out`` if given)."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 3:
        raise ValueError("x must be [T, n, C]")
    T, n, C = x.shape
    if (H is None) == (logits is None):
        raise ValueError("pass exactly one of H or logits")
    src = H if H is not None else logits
    _need(src, "H" if H is not None else "logits", torch.float32)
    if tuple(src.shape) != (T, n, n) or src.device != x.device:
        raise ValueError(f"H/logits must be [{T}, {n}, {n}] on {x.device}, got "
                         f"{tuple(src.shape)} on {src.device}")
    y = _out(out, "out", torch.bfloat16, x.shape, x.device)
    if H_out is not None and not (logits is not None and return_H):
        raise ValueError("H_out needs logits and return_H")
    if logits is not None and return_H:
        H_out = _out(H_out, "H_out", torch.float32, logits.shape, x.device)
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
    if x.dim() != 3:
        raise ValueError("x must be [T, n, C]")
    _need(grad_out, "grad_out", torch.bfloat16)
    _same(grad_out, "grad_out", x, "x")
    T, n, C = x.shape
    _need(H, "H", torch.float32)
    if tuple(H.shape) != (T, n, n) or H.device != x.device:
        raise ValueError(f"H must be [{T}, {n}, {n}] on {x.device}, got {tuple(H.shape)} on {H.device}")
    gx, gH = (None, None) if out is None else out
    gx = _out(gx, "grad_x", torch.bfloat16, x.shape, x.device)
    gH = _out(gH, "grad_H", torch.float32, H.shape, x.device)
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
    if W.device != x.device or f.device != x.device:
        raise ValueError("x, W and f must be on one device")
    a = LayerArgs()
    a.T, a.n, a.C, a.eps = T, n, C, float(eps)
    a.proj = ctypes.pointer(opts) if opts is not None else None
    a.x, a.W, a.f = x.data_ptr(), W.data_ptr(), f.data_ptr()
    return a


def _fwd_shapes(T, n, C):
    """Shapes and dtypes of the layer forward's outputs."""
    return dict(u=((T, C), torch.bfloat16), x_out=((T, n, C), torch.bfloat16),
                rms=((T,), torch.float32), logits=((T, N_MAPS), torch.float32),
                H_pre=((T, n), torch.float32), H_post=((T, n), torch.float32),
                H_res=((T, n, n), torch.float32))


def _bwd_shapes(T, n, C):
    """Shapes and dtypes of the layer backward's outputs."""
    return dict(grad_x=((T, n, C), torch.bfloat16), grad_f=((T, C), torch.bfloat16),
                grad_W=((N_MAPS, n * C), torch.float32),
                grad_logits=((T, N_MAPS), torch.float32))


def _dict_out(out, shapes, device):
    """Every tensor of a caller-provided output dict checked (or allocated)."""
    out = {} if out is None else out
    return {k: _out(out.get(k), k, dt, sh, device) for k, (sh, dt) in shapes.items()}


def layer_fwd(x, W, f, *, eps=1e-6, solver="newton", max_iters=None, tol=None,
              warm_sweeps=None, out=None):
    """Forward of one mHC layer step.  x [T,4,C], W [24,4C], f [T,C] bf16.
    Returns dict(u, x_out, rms, logits, H_pre, H_post, H_res), written into
    ``out``'s tensors when a previous result dict is passed."""
    o = make_opts(solver, max_iters, tol, warm_sweeps)
    a = _layer_args(x, W, f, eps, o)
    T, n, C = x.shape
    dev = x.device
    out = _dict_out(out, _fwd_shapes(T, n, C), dev)
    for k, t in out.items():
        setattr(a, k, t.data_ptr())
    with torch.cuda.device(dev):
        check(lib().mhc_layer_fwd(ctypes.byref(a), _stream(dev)))
    return out


def layer_fwd_into(x, W, f, out, *, eps=1e-6, solver="newton"):
    """layer_fwd writing into the tensors of a previous result dict ``out``."""
    return layer_fwd(x, W, f, eps=eps, solver=solver, out=out)


def stream_mix_into(x, logits, H_out, out, solver="newton"):
    """Fused projection + stream mix into preallocated H_out and out."""
    y, _ = stream_mix(x, logits=logits, out=out, H_out=H_out, return_H=True, solver=solver)
    return y


def layer_workspace(T, C, device, n=4):
    nbytes = lib().mhc_layer_workspace_bytes(T, n, C)
    if nbytes < 0:
        raise ValueError("invalid layer shape")
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _layer_bwd_args(x, W, f, fwd, grad_x_out, grad_u, out):
    a = _layer_args(x, W, f, 1e-6, None)
    T, n, C = x.shape
    dev = x.device
    _need(grad_x_out, "grad_x_out", torch.bfloat16)
    _same(grad_x_out, "grad_x_out", x, "x")
    _need(grad_u, "grad_u", torch.bfloat16)
    _same(grad_u, "grad_u", f, "f")
    for k, (sh, dt) in _fwd_shapes(T, n, C).items():
        if k in ("u", "x_out"):
            continue
        t = fwd[k]
        _need(t, k, dt)
        if tuple(t.shape) != sh or t.device != dev:
            raise ValueError(f"{k} must be {sh} on {dev}, got {tuple(t.shape)} on {t.device}")
        setattr(a, k, t.data_ptr())
    a.grad_x_out, a.grad_u = grad_x_out.data_ptr(), grad_u.data_ptr()
    out = _dict_out(out, _bwd_shapes(T, n, C), dev)
    for k, t in out.items():
        setattr(a, k, t.data_ptr())
    return a, out


def layer_bwd(x, W, f, fwd, grad_x_out, grad_u, *, workspace=None, out=None):
    """Backward of one mHC layer step given the forward's outputs ``fwd``.
    Returns dict(grad_x, grad_f, grad_W, grad_logits)."""
    a, out = _layer_bwd_args(x, W, f, fwd, grad_x_out, grad_u, out)
    T, n, C = x.shape
    dev = x.device
    if workspace is None:
        ws = layer_workspace(T, C, dev, n)
    else:
        ws = workspace
        _need(ws, "workspace", torch.uint8)
        if ws.device != dev:
            raise ValueError(f"workspace must be on {dev}, got {ws.device}")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    with torch.cuda.device(dev):
        check(lib().mhc_layer_bwd(ctypes.byref(a), _stream(dev)))
    return out


def layer_bwd_noalloc(x, W, f, fwd, grad_x_out, grad_u, *, out=None):
    """layer_bwd through mhc_layer_bwd_noalloc: the same result, with the
    library's own device scratch as the workspace (nothing is allocated by the
    call; pass ``out`` to allocate nothing here either).  Calls that overlap
    in time on one GPU share that scratch and race."""
    a, out = _layer_bwd_args(x, W, f, fwd, grad_x_out, grad_u, out)
    a.workspace, a.workspace_bytes = None, 0
    with torch.cuda.device(x.device):
        check(lib().mhc_layer_bwd_noalloc(ctypes.byref(a), _stream(x.device)))
    return out
