"""mhc_birkhoff_pipeline_step: the forward of one batch and the backward of
another in one launch.  P must be bit for bit mhc_birkhoff_fwd's, and the
gradient bit for bit mhc_birkhoff_bwd_recompute's for the logits whose
forward P it is given (both form it one matrix per lane), for batch sizes
that leave ragged tails in both halves and for either half empty.  Against
mhc_birkhoff_bwd (one row per lane, another summation order) the gradient
may differ only at fp32 rounding: per matrix within 1e-5 (max|dA| + max|G|),
a tenth of the oracle bar's relative part.  A sample is also compared with
the float64 oracle at the projection bars (max |dP| <= 1e-5; gradient within
1e-4 max|ref| + 1e-5 max|G|)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import birkhoff_project, birkhoff_project_bwd

pytestmark = pytest.mark.gpu


def _batch(kind, B, seed):
    A = torch.from_numpy(W.logits_batch(kind, B, seed)).cuda()
    G = torch.from_numpy(W.grad_batch(B, seed + 1)).cuda()
    return A, G


@pytest.mark.parametrize("Bf,Bb", [(3000, 5000), (5000, 3000), (1, 1), (65, 257), (257, 0),
                                   (0, 65), (4099, 1023), (1024, 1024), (20000, 20000)])
def test_pipeline_matches_separate_calls(gpu_lib, Bf, Bb):
    bp = gpu_lib
    A, _ = _batch("normal10", max(Bf, 1), 90)
    A = A[:Bf]
    Ab, Gb = _batch("normal2", max(Bb, 1), 92)
    Ab, Gb = Ab[:Bb], Gb[:Bb]
    Pb = bp.birkhoff_fwd(Ab)  # the backward batch's forward, done earlier
    P_ref, it_ref = bp.birkhoff_fwd(A, return_iters=True)
    dA_ref = bp.birkhoff_bwd_recompute(Ab, Gb)
    dA_rows = bp.birkhoff_bwd(Pb, Gb)
    P, dA, it = bp.birkhoff_pipeline_step(A, Pb, Gb, return_iters=True)
    torch.cuda.synchronize()
    assert torch.equal(P, P_ref)
    assert torch.equal(it, it_ref)
    assert torch.equal(dA, dA_ref)
    if Bb:
        _assert_rounding_close(dA, dA_rows, Gb)


def _assert_rounding_close(dA, dA_rows, G):
    d = (dA - dA_rows).abs().amax(dim=(-2, -1))
    bar = 1e-5 * (dA_rows.abs().amax(dim=(-2, -1)) + G.abs().amax(dim=(-2, -1)))
    assert bool((d <= bar).all()), f"worst {(d / bar).max().item():.2f} of the rounding bar"


def test_pipeline_against_oracle(gpu_lib):
    bp = gpu_lib
    Bf, Bb = 700, 900
    A, _ = _batch("normal10", Bf, 94)
    Ab, Gb = _batch("diag20", Bb, 96)
    Pb = bp.birkhoff_fwd(Ab)
    P, dA = bp.birkhoff_pipeline_step(A, Pb, Gb)
    torch.cuda.synchronize()
    P_or = birkhoff_project(A.cpu().numpy().astype(np.float64))
    assert np.abs(P.cpu().numpy() - P_or).max() <= 1e-5
    Pb_or = birkhoff_project(Ab.cpu().numpy().astype(np.float64))
    G64 = Gb.cpu().numpy().astype(np.float64)
    ref = birkhoff_project_bwd(Pb_or, G64)
    err = np.abs(dA.cpu().numpy() - ref).max(axis=(-2, -1))
    bar = 1e-4 * np.abs(ref).max(axis=(-2, -1)) + 1e-5 * np.abs(G64).max(axis=(-2, -1))
    assert (err <= bar).all(), f"worst {np.max(err / bar):.2f} of the bar"


def test_pipeline_aliases_and_shared_inputs(gpu_lib):
    """P may be the forward's logits and grad_logits the backward's grad_P
    (each exactly), and both halves may read the same input memory."""
    bp = gpu_lib
    B = 2000
    A, G = _batch("normal10", B, 98)
    Ab, _ = _batch("normal1", B, 100)
    Pb = bp.birkhoff_fwd(Ab)
    P_ref = bp.birkhoff_fwd(A)
    dA_ref = bp.birkhoff_bwd_recompute(Ab, G)
    # the forward batch's logits double as the backward's dL/dP (read by both)
    dA_shared_ref = bp.birkhoff_bwd_recompute(Ab, A)
    P2, dA2 = bp.birkhoff_pipeline_step(A, Pb, A)
    torch.cuda.synchronize()
    assert torch.equal(P2, P_ref) and torch.equal(dA2, dA_shared_ref)
    Ai, Gi = A.clone(), G.clone()
    bp.birkhoff_pipeline_step(Ai, Pb, Gi, out=Ai, out_grad=Gi)
    torch.cuda.synchronize()
    assert torch.equal(Ai, P_ref) and torch.equal(Gi, dA_ref)


def test_pipeline_binding_checks(gpu_lib):
    bp = gpu_lib
    A, G = _batch("normal10", 100, 102)
    Pb = bp.birkhoff_fwd(A)
    with pytest.raises(ValueError):
        bp.birkhoff_pipeline_step(A, Pb, G[:99])
    buf = torch.full((108, 4, 4), 7.0, device="cuda")
    with pytest.raises(ValueError):
        bp.birkhoff_pipeline_step(A, Pb, G, out=buf[:99])
    with pytest.raises(ValueError):
        bp.birkhoff_pipeline_step(A, Pb, G, out_grad=buf[:99])
    torch.cuda.synchronize()
    assert bool((buf == 7.0).all())


def test_pipeline_sinkhorn_solver(gpu_lib):
    """The Sinkhorn instantiation: P bit for bit birkhoff_fwd's with the same
    options (converged and fixed-count), the gradient the recompute
    backward's for the same logits and options."""
    bp = gpu_lib
    Bf, Bb = 1500, 2100
    A, _ = _batch("normal1", Bf, 104)
    Ab, Gb = _batch("normal1", Bb, 106)
    for opts in (dict(solver="sinkhorn"), dict(solver="sinkhorn", max_iters=20, tol=0.0)):
        Pb = bp.birkhoff_fwd(Ab, **opts)
        P, dA, it = bp.birkhoff_pipeline_step(A, Pb, Gb, return_iters=True, **opts)
        P_ref, it_ref = bp.birkhoff_fwd(A, return_iters=True, **opts)
        dA_ref = bp.birkhoff_bwd_recompute(Ab, Gb, **opts)
        torch.cuda.synchronize()
        assert torch.equal(P, P_ref) and torch.equal(it, it_ref), opts
        assert torch.equal(dA, dA_ref), opts


@pytest.mark.parametrize("config", [2, 3])
def test_full_size_fused_recompute_pipeline(gpu_lib, config):
    """The 131072 N(0,10^2) workload (seed 2) and the 1 M mixed one (seed 3)
    in the launch configurations bench.py times for `--fused`, `--recompute`
    and the `overlapped` figures:
    the fused launch's P and the pipeline's P bit for bit mhc_birkhoff_fwd's;
    the fused and pipeline gradients bit for bit the recompute backward's;
    the recompute gradient within fp32 rounding of mhc_birkhoff_bwd's for
    every matrix, and against the oracle on 4096 sampled matrices."""
    bp = gpu_lib
    print(f"full-size fused/recompute/pipeline, config {config}", flush=True)
    A_np, G_np = W.config2() if config == 2 else W.config3()[:2]
    A = torch.from_numpy(A_np).cuda()
    G = torch.from_numpy(G_np).cuda()
    P = bp.birkhoff_fwd(A)
    dA_rows = bp.birkhoff_bwd(P, G)
    dA_rec = bp.birkhoff_bwd_recompute(A, G)
    P_f, dA_f = bp.birkhoff_fwd_bwd(A, G)
    # pipeline: this batch's backward beside another batch's forward (the
    # same logits rolled by one matrix, a different batch of the same size)
    A2 = torch.roll(A, 1, dims=0).contiguous()
    P2_ref = bp.birkhoff_fwd(A2)
    P2, dA_p = bp.birkhoff_pipeline_step(A2, P, G)
    torch.cuda.synchronize()
    assert torch.equal(P_f, P)
    assert torch.equal(dA_f, dA_rec)
    assert torch.equal(P2, P2_ref)
    assert torch.equal(dA_p, dA_rec)
    _assert_rounding_close(dA_rec, dA_rows, G)
    idx = np.sort(np.random.Generator(np.random.PCG64(11)).choice(A_np.shape[0], 4096, replace=False))
    ref_P = birkhoff_project(A_np[idx].astype(np.float64))
    G64 = G_np[idx].astype(np.float64)
    ref = birkhoff_project_bwd(ref_P, G64)
    err = np.abs(dA_rec.cpu().numpy()[idx] - ref).max(axis=(-2, -1))
    bar = 1e-4 * np.abs(ref).max(axis=(-2, -1)) + 1e-5 * np.abs(G64).max(axis=(-2, -1))
    assert (err <= bar).all(), f"worst {np.max(err / bar):.2f} of the bar"
