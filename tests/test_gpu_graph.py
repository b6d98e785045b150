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


def test_fused_recompute_and_n8_graph_replays(gpu_lib):
    """The fused forward + backward, the recompute backward and the 8x8
    forward (whose kernel spills to scratch memory) in one captured graph."""
    B = 3000
    A = torch.from_numpy(W.logits_batch("normal10", B, 64)).cuda()
    G = torch.from_numpy(W.grad_batch(B, 65)).cuda()
    A8 = torch.from_numpy(W.logits_batch("normal10", B, 66, n=8)).cuda()
    G8 = torch.from_numpy(W.grad_batch(B, 67, n=8)).cuda()
    Pf, dAf = torch.empty_like(A), torch.empty_like(A)
    dAr = torch.empty_like(A)
    P8, dA8 = torch.empty_like(A8), torch.empty_like(A8)
    Pfe, dAfe = gpu_lib.birkhoff_fwd_bwd(A, G)
    dAre = gpu_lib.birkhoff_bwd_recompute(A, G)
    P8e = gpu_lib.birkhoff_fwd_n(A8)
    dA8e = gpu_lib.birkhoff_bwd_n(P8e, G8)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.birkhoff_fwd_bwd(A, G, out_P=Pf, out_grad=dAf)
        gpu_lib.birkhoff_bwd_recompute(A, G, out=dAr)
        gpu_lib.birkhoff_fwd_n(A8, out=P8)
        gpu_lib.birkhoff_bwd_n(P8, G8, out=dA8)
    for rep in range(3):
        for t in (Pf, dAf, dAr, P8, dA8):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Pf, Pfe) and torch.equal(dAf, dAfe), f"replay {rep}: fused"
        assert torch.equal(dAr, dAre), f"replay {rep}: recompute"
        assert torch.equal(P8, P8e) and torch.equal(dA8, dA8e), f"replay {rep}: 8x8"
        gpu_lib.birkhoff_fwd_n(A8[:100])  # eager work between replays
        torch.cuda.synchronize()


def _overlapped(gpu_lib, sets, main, side):
    """Forward of batch k on `main` while the backward of batch k-1 runs on
    `side`; the forward of batch k waits for the backward of batch k-2."""
    fwd_done = [torch.cuda.Event() for _ in sets]
    bwd_done = [torch.cuda.Event() for _ in sets]
    side.wait_stream(main)
    for k, (A, P, G, dA) in enumerate(sets):
        if k >= 2:
            main.wait_event(bwd_done[k - 2])
        gpu_lib.birkhoff_fwd(A, out=P)
        fwd_done[k].record(main)
        with torch.cuda.stream(side):
            side.wait_event(fwd_done[k])
            gpu_lib.birkhoff_bwd(P, G, out=dA)
            bwd_done[k].record(side)
    main.wait_stream(side)


def test_two_stream_overlap(gpu_lib):
    """Batches whose forward overlaps another batch's backward on a second
    stream (eagerly and in a captured graph) give the serial results bit for
    bit: the kernels share no state between launches."""
    B = 20000  # more waves than one launch keeps resident alongside the other
    sets = []
    for k in range(5):
        A = torch.from_numpy(W.logits_batch("normal10", B, 70 + k)).cuda()
        G = torch.from_numpy(W.grad_batch(B, 80 + k)).cuda()
        sets.append((A, torch.empty_like(A), G, torch.empty_like(A)))
    ref = []
    for A, P, G, dA in sets:
        Pe = gpu_lib.birkhoff_fwd(A)
        ref.append((Pe, gpu_lib.birkhoff_bwd(Pe, G)))
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def check(label):
        torch.cuda.synchronize()
        for k, ((A, P, G, dA), (Pe, dAe)) in enumerate(zip(sets, ref)):
            assert torch.equal(P, Pe), f"{label}: P of batch {k}"
            assert torch.equal(dA, dAe), f"{label}: dA of batch {k}"

    def clear():
        for A, P, G, dA in sets:
            P.fill_(float("nan"))
            dA.fill_(float("nan"))

    clear()
    _overlapped(gpu_lib, sets, main, side)
    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _overlapped(gpu_lib, sets, torch.cuda.current_stream(), side)
    torch.cuda.synchronize()
    for rep in range(3):
        clear()
        g.replay()
        check(f"replay {rep}")
        gpu_lib.birkhoff_fwd(sets[0][0][:100])  # eager work between replays
        torch.cuda.synchronize()
