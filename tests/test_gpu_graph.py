"""The C-ABI calls inside a captured HIP graph (the way the bench launches
them): every replay, with eager work and synchronisation in between, must
reproduce the eager results bit for bit.  The kernels use no memset nodes, no
allocation and no atomics, so replays are deterministic."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def test_projection_graph_replays(gpu_lib):
    B = 3000  # several workgroups and a ragged tail
    A = torch.from_numpy(W.logits_batch("normal10", B, 61)).cuda()
    G = torch.from_numpy(W.grad_batch(B, 62)).cuda()
    P = torch.empty_like(A)
    dA = torch.empty_like(A)
    Pe = gpu_lib.birkhoff_fwd(A)
    dAe = gpu_lib.birkhoff_bwd(Pe, G)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.birkhoff_fwd(A, out=P)
        gpu_lib.birkhoff_bwd(P, G, out=dA)
    for rep in range(3):
        P.fill_(float("nan"))
        dA.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(P, Pe), f"replay {rep}: P"
        assert torch.equal(dA, dAe), f"replay {rep}: dA"
        gpu_lib.birkhoff_fwd(A[:100])  # eager work between replays
        torch.cuda.synchronize()


def test_mix_graph_replays(gpu_lib):
    T, C = 200, 256
    x, logits = W.mix_inputs(T, C, seed=63)
    y = torch.empty_like(x)
    H = torch.empty_like(logits)
    ye, He = gpu_lib.stream_mix(x, logits=logits, return_H=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.ops.stream_mix_into(x, logits, H, y)
    for rep in range(3):
        y.zero_()
        H.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(H, He), f"replay {rep}: H"
        assert torch.equal(y, ye), f"replay {rep}: out"
        gpu_lib.stream_mix(x[:10], logits=logits[:10])
        torch.cuda.synchronize()
