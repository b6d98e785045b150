"""Float64 CPU oracle for the n-stream mix of mHC (forward and backward).

TEST INFRASTRUCTURE ONLY (imported by tests/, ``__graft_entry__.smoke()`` and
``bench.py``'s cpu_baseline leg; never by the product package).

The residual is widened to n parallel streams, and a learnable n x n matrix
mixes them at every layer (forpes.ru mHC explainer, section
"Hyper-Connections: more expressiveness, less stability"; neo-ai mHC summary,
section "Numerical runaway and system bottlenecks").  Applied to one token:
    out[i, :] = sum_j H[i, j] * x[j, :]
With H doubly stochastic the column sums are 1, so the sum over streams is
preserved (neo-ai summary, section "Rebuilding identity mapping with the
doubly stochastic manifold": feature means are preserved).

Backward, for upstream gradient dout:
    dx[j, :] = sum_i H[i, j] * dout[i, :]      (x's gradient)
    dH[i, j] = <dout[i, :], x[j, :]>            (H's gradient)

The bf16 inputs enter as their exact values (float64 holds every bf16); the
result is float64, not rounded.
"""
from __future__ import annotations

import numpy as np


def stream_mix(H, x):
    """out[t,i,c] = sum_j H[t,i,j] x[t,j,c], float64."""
    H = np.asarray(H, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return np.einsum("tij,tjc->tic", H, x)


def stream_mix_bwd(H, x, dout):
    """(dx, dH) of the stream mix, float64."""
    H = np.asarray(H, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    dx = np.einsum("tij,tic->tjc", H, dout)
    dH = np.einsum("tic,tjc->tij", dout, x)
    return dx, dH
