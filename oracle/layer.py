"""Float64 CPU oracle for one mHC residual-layer step (forward and backward).

TEST INFRASTRUCTURE ONLY (imported by tests/, ``__graft_entry__.smoke()`` and
``bench.py``'s cpu_baseline leg; never by the product package).

The step, per token t, as the pages describe it and with the readings this
project takes where they are silent:

* The n streams x[t] (n x C) are flattened to one vector of length D = n*C and
  RMS-normalised: r = sqrt(mean(x^2) + eps), xn = x / r, no gain (fused
  RMSNorm + matmul: neo-ai mHC summary, section "Breaking memory-bandwidth and
  communication limits").
* A dense map gives the token's dynamic logits l = xn W^T with
  W [n*n + 2n, D] (rows: pre 0:n | post n:2n | res 2n: row-major n x n); the
  mappings are generated per token (kimiseek V4-Flash article: the read,
  write and residual maps are produced from the input).
* H_pre = sigmoid(l[0:n]), H_post = sigmoid(l[n:2n]) -- non-negative through a
  sigmoid (forpes.ru explainer, section "mHC: bring back the guarantee") -- and
  H_res = P(l[2n:]), the Birkhoff projection (oracle.birkhoff).
* Read-mix into the layer function's input: u = sum_j H_pre[j] x[j].
* Write-back: x_out[i] = H_post[i] f + sum_j H_res[i, j] x[j], f being the
  layer function's output (forpes.ru explainer, section "Hyper-Connections":
  the widened stream is projected down before F and expanded after).

Backward for upstream (dx_out, du), by the chain rule in float64, with the
projection's gradient from oracle.birkhoff.birkhoff_project_bwd.

Pins (tests/test_oracle_mix_layer.py): the forward by closed forms on one-hot
maps W (logit m = x_k / r, sigmoid maps, and the projection of a matrix with
one nonzero entry, solved by symmetry), by the scale invariance of the
normalised logits, and u / x_out by explicit loops; the backward by central
finite differences of a scalar loss and by torch float64 autograd through
unrolled Sinkhorn sweeps.
"""
from __future__ import annotations

import numpy as np

from .birkhoff import birkhoff_project, birkhoff_project_bwd

EPS = 1e-6


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def layer_fwd(x, W, f, eps=EPS, streams=True):
    """Forward of the layer step.  x [T,n,C], W [n*n+2n, n*C], f [T,C].
    Returns a dict with float64 arrays: rms [T], logits [T, n*n+2n],
    H_pre [T,n], H_post [T,n], H_res [T,n,n], u [T,C], x_out [T,n,C].
    With ``streams`` False, u and x_out are left out (the rest is computed
    exactly as with them)."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    f = np.asarray(f, dtype=np.float64)
    T, n, C = x.shape
    D = n * C
    xf = x.reshape(T, D)
    rms = np.sqrt((xf * xf).mean(axis=1) + eps)
    xn = xf / rms[:, None]
    logits = xn @ W.T
    H_pre = _sigmoid(logits[:, :n])
    H_post = _sigmoid(logits[:, n:2 * n])
    H_res = birkhoff_project(logits[:, 2 * n:].reshape(T, n, n))
    if not streams:
        return dict(rms=rms, logits=logits, H_pre=H_pre, H_post=H_post, H_res=H_res)
    u = np.einsum("tj,tjc->tc", H_pre, x)
    x_out = H_post[:, :, None] * f[:, None, :] + np.einsum("tij,tjc->tic", H_res, x)
    return dict(rms=rms, logits=logits, H_pre=H_pre, H_post=H_post,
                H_res=H_res, u=u, x_out=x_out)


def layer_bwd(x, W, f, dx_out, du, fwd=None, eps=EPS, streams=True):
    """Backward of the layer step for upstream gradients dx_out [T,n,C] and
    du [T,C].  Returns dict(dx [T,n,C], dW [n*n+2n, n*C], df [T,C],
    dlogits [T, n*n+2n]).  With ``streams`` False, dx and df are left out
    (dW and dlogits are computed exactly as with them)."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    f = np.asarray(f, dtype=np.float64)
    dx_out = np.asarray(dx_out, dtype=np.float64)
    du = np.asarray(du, dtype=np.float64)
    if fwd is None:
        fwd = layer_fwd(x, W, f, eps)
    T, n, C = x.shape
    D = n * C
    H_pre, H_post, H_res, rms = fwd["H_pre"], fwd["H_post"], fwd["H_res"], fwd["rms"]
    # write-back and read-mix
    dH_post = np.einsum("tic,tc->ti", dx_out, f)
    dH_res = np.einsum("tic,tjc->tij", dx_out, x)
    dH_pre = np.einsum("tc,tjc->tj", du, x)
    # maps -> logits
    dl_pre = dH_pre * H_pre * (1.0 - H_pre)
    dl_post = dH_post * H_post * (1.0 - H_post)
    dl_res = birkhoff_project_bwd(H_res, dH_res).reshape(T, n * n)
    dl = np.concatenate([dl_pre, dl_post, dl_res], axis=1)
    # logits = xn W^T
    xf = x.reshape(T, D)
    xn = xf / rms[:, None]
    dW = dl.T @ xn
    if not streams:
        return dict(dW=dW, dlogits=dl)
    df = np.einsum("ti,tic->tc", H_post, dx_out)
    dx = np.einsum("tij,tic->tjc", H_res, dx_out) + H_pre[:, :, None] * du[:, None, :]
    dxn = dl @ W
    # xn = x / sqrt(mean(x^2) + eps)
    proj = (dxn * xn).sum(axis=1) / D
    dx_norm = (dxn - xn * proj[:, None]) / rms[:, None]
    dx = dx + dx_norm.reshape(T, n, C)
    return dict(dx=dx, dW=dW, df=df, dlogits=dl)
