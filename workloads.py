"""Seeded synthetic inputs for the mHC Birkhoff-projection workloads.

This module only draws random numbers and arranges them into the shapes the
workloads use.  It holds none of the method's arithmetic (no exp, no
normalisation, no projection), so both the float64 oracle and the HIP path can
take their inputs from it without sharing any computation.

Distributions follow the accuracy study of "Accelerating Birkhoff projection for
mHC" (gist.science summary, section 4 "Experimental results": small-magnitude
N(0,1) and large-magnitude N(0,10^2) inputs) and the mHC layer description
(n = 4 residual streams; forpes.ru explainer, section "Hyper-Connections").

Conventions
-----------
* CPU draws: ``numpy.random.Generator(PCG64(seed))`` standard normals in float64,
  scaled, then rounded to float32 (round-to-nearest-even, numpy's cast).
* Large bf16 tensors (stream mix, full layer) are drawn on the device with a
  seeded ``torch.Generator`` in float32 and rounded to bfloat16 (RNE, torch's
  cast).  Token subsets are copied back for the oracle.
"""
from __future__ import annotations

import numpy as np

N_STREAMS = 4

# name -> (B or T, description); the parity tests also use smaller batches of
# the same distributions.
PROJ_KINDS = ("normal1", "normal10", "diag20")


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def logits_batch(kind: str, B: int, seed: int, n: int = N_STREAMS) -> np.ndarray:
    """[B,n,n] float32 logits of one distribution.

    kind: "normal1"  -> N(0,1)
          "normal10" -> N(0,10^2)
          "diag20"   -> N(0,1) plus 20 on the diagonal (near-identity case)
          "normal2"  -> N(0,2^2) (the fused stream-mix workload's logits)
    """
    g = _rng(seed)
    z = g.standard_normal((B, n, n))
    if kind == "normal1":
        a = z
    elif kind == "normal10":
        a = 10.0 * z
    elif kind == "normal2":
        a = 2.0 * z
    elif kind == "diag20":
        a = z + 20.0 * np.eye(n)[None]
    else:
        raise ValueError(f"unknown logits kind {kind!r}")
    return a.astype(np.float32)


def grad_batch(B: int, seed: int, n: int = N_STREAMS) -> np.ndarray:
    """[B,n,n] float32 upstream gradient dL/dP, N(0,1)."""
    return _rng(seed).standard_normal((B, n, n)).astype(np.float32)


def mixed_batch(B: int, seed: int, n: int = N_STREAMS):
    """Mixed-difficulty batch: 50% N(0,1), 40% N(0,10^2), 10% N(0,1)+20*I,
    concatenated in that order, then permuted by the seed; then the upstream
    gradient N(0,1) from the same generator.  Returns (A, G, kind_index) where
    kind_index[b] is 0/1/2 for the three distributions.
    """
    g = _rng(seed)
    b1 = B // 2
    b2 = (B * 2) // 5
    b3 = B - b1 - b2
    z = g.standard_normal((B, n, n))
    a = np.empty((B, n, n))
    a[:b1] = z[:b1]
    a[b1:b1 + b2] = 10.0 * z[b1:b1 + b2]
    a[b1 + b2:] = z[b1 + b2:] + 20.0 * np.eye(n)[None]
    kind = np.concatenate([np.zeros(b1, np.int8), np.ones(b2, np.int8),
                           np.full(b3, 2, np.int8)])
    perm = g.permutation(B)
    a = a[perm]
    kind = kind[perm]
    G = g.standard_normal((B, n, n))
    return a.astype(np.float32), G.astype(np.float32), kind


# ---------------------------------------------------------------------------
# The five workload configurations (sizes and seeds).
# ---------------------------------------------------------------------------

def config1():
    """Forward only: 4096 matrices N(0,1), seed 0."""
    return logits_batch("normal1", 4096, 0)


def config2():
    """Forward+backward: 131072 matrices N(0,10^2) then G N(0,1), one
    generator seeded 2 (A drawn first, then G)."""
    g = _rng(2)
    A = (10.0 * g.standard_normal((131072, 4, 4))).astype(np.float32)
    G = g.standard_normal((131072, 4, 4)).astype(np.float32)
    return A, G


def config3():
    """Mixed difficulty, 1,048,576 matrices, seed 3: 524288 N(0,1),
    419430 N(0,10^2), 104858 N(0,1)+20I, shuffled; G N(0,1)."""
    return mixed_batch(1048576, 3)


CONFIG4_SHAPE = dict(T=16384, n=4, C=4096)
CONFIG5_SHAPE = dict(T=65536, n=4, C=7168)


def _torch_gen(seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def _randn_bf16(shape, gen, device, scale=1.0, chunk_rows=4096):
    """N(0, scale^2) drawn in float32 by ``gen`` then rounded to bf16.  Drawn
    in chunks over the leading dim so that the float32 staging stays small."""
    import torch
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        t = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen,
                        dtype=torch.float32, device=device)
        if scale != 1.0:
            t.mul_(scale)
        out[r0:r1].copy_(t)
    return out


def mix_inputs(T: int, C: int, seed: int = 4, device="cuda", n: int = N_STREAMS,
               logit_scale: float = 2.0):
    """Fused projection + stream mix inputs: x [T,n,C] bf16 N(0,1) and
    logits [T,n,n] fp32 N(0, logit_scale^2), drawn in that order."""
    import torch
    gen = _torch_gen(seed, device)
    x = _randn_bf16((T, n, C), gen, device)
    logits = torch.randn((T, n, n), generator=gen, dtype=torch.float32,
                         device=device) * logit_scale
    return x, logits


def mix_bwd_inputs(T: int, C: int, seed: int = 40, device="cuda", n: int = N_STREAMS):
    """Stream-mix backward inputs: x, dout [T,n,C] bf16 N(0,1) and a mixing
    matrix source: logits [T,n,n] fp32 N(0,2^2) (projected by the caller)."""
    import torch
    gen = _torch_gen(seed, device)
    x = _randn_bf16((T, n, C), gen, device)
    dout = _randn_bf16((T, n, C), gen, device)
    logits = torch.randn((T, n, n), generator=gen, dtype=torch.float32,
                         device=device) * 2.0
    return x, dout, logits


def layer_inputs(T: int, C: int, seed: int = 5, device="cuda", n: int = N_STREAMS,
                 w_scale: float = 0.02):
    """Full mHC layer inputs, drawn in this order from one generator:
    x [T,n,C] bf16 N(0,1); W [n*n+2n, n*C] bf16 N(0, w_scale^2) (rows are the
    dynamic-map outputs: pre 0:n | post n:2n | res 2n: row-major n x n);
    f [T,C] bf16 N(0,1); upstream dx_out [T,n,C] and du [T,C] bf16 N(0,1)."""
    gen = _torch_gen(seed, device)
    x = _randn_bf16((T, n, C), gen, device)
    W = _randn_bf16((n * n + 2 * n, n * C), gen, device, scale=w_scale)
    f = _randn_bf16((T, C), gen, device)
    dx_out = _randn_bf16((T, n, C), gen, device)
    du = _randn_bf16((T, C), gen, device)
    return dict(x=x, W=W, f=f, dx_out=dx_out, du=du)
