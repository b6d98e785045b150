"""GPU parity of the n x n projection (1 <= n <= 8, mhc_birkhoff_fwd_n /
mhc_birkhoff_bwd_n) against the float64 oracle, which is written for any n.
Same bars as the 4x4 tests (test_gpu_birkhoff.py)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import birkhoff_project, birkhoff_project_bwd

pytestmark = pytest.mark.gpu

P_TOL = 1e-5
SUM_TOL = 1e-5


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _fwd(bp, A, **kw):
    P, it = bp.birkhoff_fwd_n(_t(A), return_iters=True, **kw)
    torch.cuda.synchronize()
    return P.cpu().numpy(), it.cpu().numpy()


def _bwd(bp, P, G):
    dA = bp.birkhoff_bwd_n(_t(P), _t(G))
    torch.cuda.synchronize()
    return dA.cpu().numpy()


def _check(P, dA, A, G, label):
    ref = birkhoff_project(A.astype(np.float64))
    P64 = P.astype(np.float64)
    err = np.abs(P64 - ref).max()
    assert err <= P_TOL, f"{label}: P error {err:.3e}"
    assert (P >= 0).all(), label
    assert np.abs(P64.sum(-1) - 1).max() <= SUM_TOL, label
    assert np.abs(P64.sum(-2) - 1).max() <= SUM_TOL, label
    dref = birkhoff_project_bwd(ref, G.astype(np.float64))
    tol = 1e-4 * np.abs(dref).max(axis=(-2, -1)) + 1e-5 * np.abs(G).max(axis=(-2, -1))
    ratio = (np.abs(dA.astype(np.float64) - dref).max(axis=(-2, -1)) / tol).max()
    assert ratio <= 1.0, f"{label}: gradient error {ratio:.3f} x tolerance"


@pytest.mark.parametrize("n", [2, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("kind", ["normal1", "normal10", "diag20"])
def test_fwd_bwd_n(gpu_lib, n, kind):
    print(f"n={n} kind={kind}", flush=True)
    B = 600  # two full workgroups and a ragged one
    A = W.logits_batch(kind, B, 500 + 10 * n, n=n)
    G = W.grad_batch(B, 600 + 10 * n, n=n)
    P, it = _fwd(gpu_lib, A)
    assert (it == 255).sum() <= 0.005 * B
    _check(P, _bwd(gpu_lib, P, G), A, G, f"n={n} {kind}")


def test_n2_closed_form(gpu_lib):
    """2x2: P = [[p, 1-p], [1-p, p]], p = sigmoid((a11 + a22 - a12 - a21) / 2)."""
    A = W.logits_batch("normal10", 1000, 71, n=2).astype(np.float64) / 3.0
    P, _ = _fwd(gpu_lib, A)
    s = A[:, 0, 0] + A[:, 1, 1] - A[:, 0, 1] - A[:, 1, 0]
    p = 1.0 / (1.0 + np.exp(-s / 2))
    want = np.stack([np.stack([p, 1 - p], -1), np.stack([1 - p, p], -1)], -2)
    assert np.abs(P - want).max() <= 1e-6


def test_n4_routes_to_4x4_kernels(gpu_lib):
    A = _t(W.logits_batch("normal10", 333, 72))
    G = _t(W.grad_batch(333, 73))
    P4 = gpu_lib.birkhoff_fwd(A)
    Pn = gpu_lib.birkhoff_fwd_n(A)
    torch.cuda.synchronize()
    assert torch.equal(P4, Pn)
    assert torch.equal(gpu_lib.birkhoff_bwd(P4, G), gpu_lib.birkhoff_bwd_n(P4, G))


def test_n1_and_sinkhorn_and_alias(gpu_lib):
    A1 = _t(np.random.default_rng(3).standard_normal((50, 1, 1)))
    P1 = gpu_lib.birkhoff_fwd_n(A1)
    torch.cuda.synchronize()
    assert torch.equal(P1, torch.ones_like(P1))
    assert torch.equal(gpu_lib.birkhoff_bwd_n(P1, A1), torch.zeros_like(P1))
    for n in (3, 8):
        A = W.logits_batch("normal1", 500, 74 + n, n=n)
        P, it = _fwd(gpu_lib, A, solver="sinkhorn", tol=1e-6, max_iters=1000)
        assert (it != 255).all()
        assert np.abs(P.astype(np.float64) - birkhoff_project(A.astype(np.float64))).max() <= P_TOL
        # P may be written over the logits, dA over the gradient
        At = _t(A)
        want = gpu_lib.birkhoff_fwd_n(At)
        gpu_lib.birkhoff_fwd_n(At, out=At)
        G = _t(W.grad_batch(500, 80 + n, n=n))
        dwant = gpu_lib.birkhoff_bwd_n(want, G)
        gpu_lib.birkhoff_bwd_n(want, G, out=G)
        torch.cuda.synchronize()
        assert torch.equal(At, want) and torch.equal(G, dwant)


def test_n2_generic_path_matches_closed_form(gpu_lib):
    """Buffers 4 bytes off a 16-byte boundary take the generic Newton kernel
    for n = 2; it must agree with the closed-form kernel."""
    B = 700
    A = W.logits_batch("normal10", B, 91, n=2)
    G = W.grad_batch(B, 92, n=2)
    P_closed = gpu_lib.birkhoff_fwd_n(_t(A))
    dA_closed = gpu_lib.birkhoff_bwd_n(P_closed, _t(G))

    def offset(a):
        buf = torch.zeros(a.size + 1, dtype=torch.float32, device="cuda")
        v = buf[1:].view(a.shape)
        v.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))
        return v
    Ao, Go = offset(A), offset(G)
    Po = offset(np.zeros_like(A))
    gpu_lib.birkhoff_fwd_n(Ao, out=Po)
    dAo = offset(np.zeros_like(A))
    gpu_lib.birkhoff_bwd_n(Po, Go, out=dAo)
    torch.cuda.synchronize()
    assert (Ao.data_ptr() % 16) != 0
    assert (Po - P_closed).abs().max().item() <= 2e-6
    tol = 1e-4 * dA_closed.abs().amax(dim=(1, 2)) + 1e-5 * torch.from_numpy(np.abs(G)).cuda().amax(dim=(1, 2))
    assert ((dAo - dA_closed).abs().amax(dim=(1, 2)) <= tol).all()


@pytest.mark.parametrize("n", [3, 5, 6])
def test_assignment_start_keeps_newton_short(gpu_lib, n):
    """For 3 <= n <= 6 Newton starts from the assignment problem's dual: on
    16384 N(0,10^2) matrices every matrix converges within 9 Newton
    iterations (a CPU replay of the kernel code needs at most 7; from g = 0
    and one Sinkhorn sweep it needed up to 21), and results match the
    oracle on a sample."""
    print(f"assignment start n={n}", flush=True)
    A = W.logits_batch("normal10", 16384, 900 + n, n=n)
    P, it = _fwd(gpu_lib, A)
    assert (it != 255).all()
    assert it.max() <= 9, f"n={n}: {it.max()} Newton iterations"
    ref = birkhoff_project(A[:512].astype(np.float64))
    assert np.abs(P[:512].astype(np.float64) - ref).max() <= P_TOL


@pytest.mark.parametrize("n", [3, 5, 6, 7, 8])
def test_fwd_bwd_n_full_size(gpu_lib, n):
    """The n x n workload `bench.py --config 2 --n N` times: 131072
    N(0,10^2) matrices (seed 2) and N(0,1) gradients (seed 3), one launch
    each way.  Every output is checked for the doubly-stochastic properties;
    a seeded sample of 1024 matrices, and every matrix flagged as not
    converged, against the oracle forward and backward at the usual bars.
    At most 0.05 % of the matrices may be flagged (a flag means the fp32
    noise floor or the line search stopped the solve above tol)."""
    print(f"general-n full size n={n}", flush=True)
    B = 131072
    A = W.logits_batch("normal10", B, 2, n=n)
    G = W.grad_batch(B, 3, n=n)
    P, it = _fwd(gpu_lib, A)
    dA = _bwd(gpu_lib, P, G)
    flagged = np.flatnonzero(it == 255)
    assert flagged.size <= 0.0005 * B, f"n={n}: {flagged.size} flagged"
    P64 = P.astype(np.float64)
    assert (P >= 0).all()
    assert np.abs(P64.sum(-1) - 1).max() <= SUM_TOL
    assert np.abs(P64.sum(-2) - 1).max() <= SUM_TOL
    assert np.isfinite(dA).all()
    idx = np.union1d(np.random.default_rng(1000 + n).choice(B, 1024, replace=False), flagged)
    _check(P[idx], dA[idx], A[idx], G[idx], f"n={n} full size, {idx.size} sampled")



@pytest.mark.parametrize("n", [3, 8])
def test_tolerance_option_n(gpu_lib, n):
    """opts.tol for the n x n solver, as for the 4x4 one: loose tol converges
    with column sums within it; tol below the fp32 floor ends flagged at the
    noise floor with P within the oracle bars."""
    A = W.logits_batch("normal10", 1000, 46 + n, n=n)
    P, it = _fwd(gpu_lib, A, tol=1e-3)
    assert (it != 255).all()
    P64 = P.astype(np.float64)
    assert np.abs(P64.sum(-2) - 1).max() <= 1e-3 * 1.0001 + 1e-6
    assert np.abs(P64.sum(-1) - 1).max() <= SUM_TOL
    P9, it9 = _fwd(gpu_lib, A, tol=1e-9)
    assert (it9 == 255).mean() > 0.5
    ref = birkhoff_project(A.astype(np.float64))
    assert np.abs(P9.astype(np.float64) - ref).max() <= P_TOL
    assert np.abs(P9.astype(np.float64).sum(-2) - 1).max() <= SUM_TOL
