"""Pins for the float64 projection oracle (oracle/birkhoff.py).

Each test checks the oracle against something other than itself: a closed
form, an invariant of doubly stochastic matrices that the pages state, an
independent 50-digit solve, finite differences, or autograd through unrolled
Sinkhorn sweeps.  No GPU.
"""
import math

import numpy as np
import pytest

import workloads
from oracle.birkhoff import (birkhoff_project, birkhoff_project_bwd, residual,
                             sinkhorn, sinkhorn_fixed)


def _p2(A2):
    """2x2 closed form: with r = K11 K22 / (K12 K21), the projection is
    [[p, 1-p], [1-p, p]] with p = sqrt(r) / (1 + sqrt(r)) = sigmoid(s/2),
    s = A11 + A22 - A12 - A21."""
    s = A2[..., 0, 0] + A2[..., 1, 1] - A2[..., 0, 1] - A2[..., 1, 0]
    p = 1.0 / (1.0 + np.exp(-s / 2.0))
    out = np.empty(A2.shape)
    out[..., 0, 0] = p
    out[..., 1, 1] = p
    out[..., 0, 1] = 1 - p
    out[..., 1, 0] = 1 - p
    return out


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# forward: closed forms
# --------------------------------------------------------------------------

def test_fwd_2x2_closed_form():
    A = _rng(10).standard_normal((500, 2, 2)) * 3.0
    P = birkhoff_project(A)
    np.testing.assert_allclose(P, _p2(A), atol=1e-13, rtol=0)


def test_fwd_2x2_sqrt_ratio_form():
    # the same closed form written with the ratio of products of K entries
    A = _rng(11).standard_normal((200, 2, 2))
    K = np.exp(A)
    r = K[:, 0, 0] * K[:, 1, 1] / (K[:, 0, 1] * K[:, 1, 0])
    p = np.sqrt(r) / (1 + np.sqrt(r))
    P = birkhoff_project(A)
    np.testing.assert_allclose(P[:, 0, 0], p, atol=1e-13)
    np.testing.assert_allclose(P[:, 0, 1], 1 - p, atol=1e-13)


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_fwd_kronecker_4x4(scale):
    """A[2a+b, 2c+d] = A1[a,c] + A2[b,d]  =>  K = K1 (x) K2 and, by uniqueness
    of the diagonal scaling, P = P2(A1) (x) P2(A2)."""
    g = _rng(12)
    A1 = g.standard_normal((100, 2, 2)) * scale
    A2 = g.standard_normal((100, 2, 2)) * scale
    A = (A1[:, :, None, :, None] + A2[:, None, :, None, :]).reshape(100, 4, 4)
    want = np.einsum("bac,bxy->baxcy", _p2(A1), _p2(A2)).reshape(100, 4, 4)
    np.testing.assert_allclose(birkhoff_project(A), want, atol=1e-13)


def test_fwd_circulant_is_row_softmax():
    """A[i,j] = c[(j-i) mod 4]: every row and every column of exp(A) holds the
    same values, so the row softmax is already doubly stochastic."""
    c = _rng(13).standard_normal((100, 4)) * 3
    idx = (np.arange(4)[None, :] - np.arange(4)[:, None]) % 4
    A = c[:, idx]
    E = np.exp(A)
    want = E / E.sum(axis=2, keepdims=True)
    np.testing.assert_allclose(birkhoff_project(A), want, atol=1e-13)


def test_fwd_rank_one_kernel_gives_uniform():
    """K = exp(u 1^T + 1 v^T) has rank one; its scaling is the uniform J/4."""
    g = _rng(14)
    u = g.standard_normal((50, 4, 1)) * 5
    v = g.standard_normal((50, 1, 4)) * 5
    P = birkhoff_project(u + v)
    np.testing.assert_allclose(P, np.full((50, 4, 4), 0.25), atol=1e-13)


@pytest.mark.parametrize("t", [-3.0, 0.0, math.log(3.0), 2.5, 20.0])
def test_fwd_scaled_identity(t):
    """A = t I: by symmetry P = a I + b (J - I) with a + 3b = 1 and
    a / b = e^t, so a = e^t / (e^t + 3), b = 1 / (e^t + 3)."""
    P = birkhoff_project(t * np.eye(4))
    a = math.exp(t) / (math.exp(t) + 3)
    b = 1 / (math.exp(t) + 3)
    np.testing.assert_allclose(P, b + (a - b) * np.eye(4), atol=1e-13)


@pytest.mark.parametrize("off", [-30.0, -200.0])
def test_fwd_block_diagonal(off):
    """Two 2x2 blocks with very negative off-block logits: P is the two 2x2
    projections on the diagonal blocks (off-block mass of order e^off)."""
    g = _rng(15)
    A1 = g.standard_normal((40, 2, 2))
    A2 = g.standard_normal((40, 2, 2))
    A = np.full((40, 4, 4), off)
    A[:, :2, :2] = A1
    A[:, 2:, 2:] = A2
    want = np.zeros((40, 4, 4))
    want[:, :2, :2] = _p2(A1)
    want[:, 2:, 2:] = _p2(A2)
    np.testing.assert_allclose(birkhoff_project(A), want, atol=1e-11)


def test_fwd_one_by_one_is_one():
    """n = 1: the doubly stochastic condition leaves the scalar 1 (neo-ai mHC
    summary: with expansion rate 1 the map falls back to the identity)."""
    A = _rng(16).standard_normal((10, 1, 1)) * 7
    np.testing.assert_array_equal(birkhoff_project(A), np.ones((10, 1, 1)))


# --------------------------------------------------------------------------
# forward: invariants of the doubly stochastic set and of the scaling
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def hard_batch():
    A = np.concatenate([workloads.logits_batch("normal1", 300, 20),
                        workloads.logits_batch("normal10", 300, 21),
                        workloads.logits_batch("diag20", 100, 22)]).astype(np.float64)
    return A, birkhoff_project(A)


def test_fwd_doubly_stochastic(hard_batch):
    A, P = hard_batch
    assert (P >= 0).all()
    assert residual(P).max() < 1e-13


def test_fwd_shift_invariance(hard_batch):
    """Adding u 1^T + 1 v^T to A changes only the scaling vectors."""
    A, P = hard_batch
    g = _rng(17)
    A2 = A + g.standard_normal((A.shape[0], 4, 1)) * 5 + g.standard_normal((A.shape[0], 1, 4)) * 5
    np.testing.assert_allclose(birkhoff_project(A2), P, atol=1e-11)


def test_fwd_permutation_equivariance(hard_batch):
    A, P = hard_batch
    g = _rng(18)
    p1, p2 = g.permutation(4), g.permutation(4)
    P2 = birkhoff_project(A[:, p1][:, :, p2])
    np.testing.assert_allclose(P2, P[:, p1][:, :, p2], atol=1e-11)


def test_fwd_transpose_equivariance(hard_batch):
    A, P = hard_batch
    np.testing.assert_allclose(birkhoff_project(np.swapaxes(A, 1, 2)),
                               np.swapaxes(P, 1, 2), atol=1e-11)


def test_fwd_spectral_norm_and_products(hard_batch):
    """Spectral norm of a doubly stochastic matrix is 1 (the all-ones vector
    is a singular vector), and products stay doubly stochastic (neo-ai
    summary: norm preservation and closure under composition)."""
    _, P = hard_batch
    s = np.linalg.svd(P, compute_uv=False)
    np.testing.assert_allclose(s[:, 0], 1.0, atol=1e-12)
    prod = P[:100] @ P[100:200] @ P[200:300]
    assert residual(prod).max() < 1e-12
    assert (prod >= 0).all()


def test_fwd_mean_preservation(hard_batch):
    """Column sums 1: the sum over streams of P x equals the sum of x."""
    _, P = hard_batch
    x = _rng(19).standard_normal((P.shape[0], 4, 7))
    np.testing.assert_allclose((P @ x).sum(axis=1), x.sum(axis=1), atol=1e-11)


def test_fwd_near_identity():
    """Strongly diagonal logits give P close to the identity (Deep Signal mHC
    article: I is in the polytope, so a near-identity start behaves like a
    plain residual)."""
    A = workloads.logits_batch("diag20", 200, 23)
    P = birkhoff_project(A)
    assert np.abs(P - np.eye(4)).max() < 1e-6


def test_fwd_sinkhorn_fixed_point(hard_batch):
    """One more Sinkhorn sweep on the result changes it by < 1e-12."""
    _, P = hard_batch
    Q = P / P.sum(axis=2, keepdims=True)
    Q = Q / Q.sum(axis=1, keepdims=True)
    assert np.abs(Q - P).max() < 1e-12


def _mp_semidual_root(A_row, P_start, dps=50):
    """Independent 50-digit solve: find column potentials g (g_3 = 0) with
    the row softmax of A + 1 g^T having unit column sums (mpmath findroot),
    started from the oracle's answer."""
    import mpmath as mp
    with mp.workdps(dps):
        A_ = [[mp.mpf(float(v)) for v in row] for row in A_row]
        n = len(A_)

        def Pmat(gs):
            g = list(gs) + [mp.mpf(0)]
            out = []
            for i in range(n):
                z = [A_[i][j] + g[j] for j in range(n)]
                m = max(z)
                e = [mp.e ** (v - m) for v in z]
                s = sum(e)
                out.append([v / s for v in e])
            return out

        def F(*gs):
            P = Pmat(gs)
            return [sum(P[i][j] for i in range(n)) - 1 for j in range(n - 1)]

        # starting guess from the oracle: P_ij / P_i3 = exp(A_ij - A_i3 + g_j)
        g0 = [mp.mpf(float(np.mean(np.log(P_start[:, j]) - np.log(P_start[:, n - 1])
                                   - (np.asarray(A_row)[:, j] - np.asarray(A_row)[:, n - 1]))))
              for j in range(n - 1)]
        root = mp.findroot(F, g0, tol=mp.mpf(10) ** (-40), maxsteps=200)
        P = Pmat([root[j] for j in range(n - 1)])
        return np.array([[float(P[i][j]) for j in range(n)] for i in range(n)])


@pytest.mark.parametrize("kind,seed", [("normal1", 30), ("normal10", 31), ("diag20", 32)])
def test_fwd_mpmath_brute_force(kind, seed):
    A = workloads.logits_batch(kind, 12, seed).astype(np.float64)
    P = birkhoff_project(A)
    for b in range(A.shape[0]):
        ref = _mp_semidual_root(A[b], P[b])
        assert np.abs(P[b] - ref).max() < 1e-12, (kind, b)


def test_fwd_mpmath_fallback_path():
    """Force every matrix through the oracle's 50-digit fallback (one Sinkhorn
    sweep, no float64 Newton) and compare with the normal path."""
    A = workloads.logits_batch("normal10", 4, 33).astype(np.float64)
    P_fb, info = birkhoff_project(A, max_sweeps=1, newton_iters=0, return_info=True)
    assert info["mp"].all()
    np.testing.assert_allclose(P_fb, birkhoff_project(A), atol=1e-12)


def test_fwd_newton_polish_path():
    """Force the float64 two-sided Newton on N(0,1) inputs (Sinkhorn capped
    at 2 sweeps) and compare with plain Sinkhorn to 1e-13."""
    A = workloads.logits_batch("normal1", 200, 34).astype(np.float64)
    P_n, info = birkhoff_project(A, max_sweeps=2, return_info=True)
    assert info["polished"].all() and not info["mp"].any()
    P_sk, _, _, _, conv = sinkhorn(A, max_sweeps=5000)
    assert conv.all()
    np.testing.assert_allclose(P_n, P_sk, atol=1e-12)


def test_fixed_sweeps_inaccurate_on_large_inputs():
    """Fixed 20-sweep Sinkhorn is accurate on N(0,1) but not on N(0,10^2)
    (summary, section 1 item 3 and section 4, accuracy)."""
    A1 = workloads.logits_batch("normal1", 500, 35)
    A10 = workloads.logits_batch("normal10", 500, 36)
    e1 = np.abs(sinkhorn_fixed(A1, 20) - birkhoff_project(A1)).max(axis=(1, 2))
    e10 = np.abs(sinkhorn_fixed(A10, 20) - birkhoff_project(A10)).max(axis=(1, 2))
    assert np.median(e1) < 1e-6
    assert np.median(e10) > 100 * np.median(e1)


def test_fixed_sweeps_exact_values():
    """sinkhorn_fixed against hand-derived exact rationals after 1, 2 and 3
    sweeps (tests/golden/closed_forms.json, 'sinkhorn_fixed_cases'): a sweep
    divides rows by their sums, then columns (Deep Signal article,
    Sinkhorn-Knopp section).  A columns-first order, one sweep more or fewer,
    or a transposed operand each fail one of them."""
    import json
    import os
    from fractions import Fraction
    path = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")
    with open(path) as fh:
        cases = json.load(fh)["sinkhorn_fixed_cases"]
    assert len(cases) >= 5
    for case in cases:
        A = np.log(np.array(case["K"], dtype=np.float64))
        want = np.array([[float(Fraction(v)) for v in row] for row in case["P"]])
        got = sinkhorn_fixed(A[None], case["sweeps"])[0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14, err_msg=case["name"])
    # the batch dimension is independent: the cases stacked give the same values
    sq = [c for c in cases if len(c["K"]) == 4 and c["sweeps"] == 1]
    A = np.log(np.array([c["K"] for c in sq], dtype=np.float64))
    want = np.array([[[float(Fraction(v)) for v in row] for row in c["P"]] for c in sq])
    np.testing.assert_allclose(sinkhorn_fixed(A, 1), want, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def test_bwd_2x2_closed_form():
    """With p = sigmoid(s/2), s = A11 + A22 - A12 - A21, and L = <G, P>,
    dL/dA = (G11 - G12 - G21 + G22) p (1-p) / 2 * [[1,-1],[-1,1]]."""
    g = _rng(40)
    A = g.standard_normal((300, 2, 2)) * 2
    G = g.standard_normal((300, 2, 2))
    P = birkhoff_project(A)
    p = P[:, 0, 0]
    k = (G[:, 0, 0] - G[:, 0, 1] - G[:, 1, 0] + G[:, 1, 1]) * p * (1 - p) / 2
    want = k[:, None, None] * np.array([[1.0, -1.0], [-1.0, 1.0]])
    np.testing.assert_allclose(birkhoff_project_bwd(P, G), want, atol=1e-13)


@pytest.mark.parametrize("kind,scale", [("normal1", 1.0), ("normal10", 0.3)])
def test_bwd_finite_differences(kind, scale):
    """Central differences of L(A) = <G, P(A)>, h = 1e-6, float64."""
    g = _rng(41)
    A = g.standard_normal((6, 4, 4)) * (10 * scale if kind == "normal10" else 1.0)
    G = g.standard_normal((6, 4, 4))
    dA = birkhoff_project_bwd(birkhoff_project(A), G)
    h = 1e-6
    fd = np.zeros_like(A)
    for i in range(4):
        for j in range(4):
            Ap = A.copy()
            Am = A.copy()
            Ap[:, i, j] += h
            Am[:, i, j] -= h
            fd[:, i, j] = ((birkhoff_project(Ap) - birkhoff_project(Am)) * G).sum(axis=(1, 2)) / (2 * h)
    np.testing.assert_allclose(dA, fd, atol=2e-8)


def test_bwd_invariants(hard_batch):
    A, P = hard_batch
    g = _rng(42)
    G1 = g.standard_normal(P.shape)
    G2 = g.standard_normal(P.shape)
    d1 = birkhoff_project_bwd(P, G1)
    d2 = birkhoff_project_bwd(P, G2)
    # P is invariant to row/column shifts of A, so dA has zero row/col sums
    assert np.abs(d1.sum(axis=1)).max() < 1e-13
    assert np.abs(d1.sum(axis=2)).max() < 1e-13
    # G = u 1^T + 1 v^T is orthogonal to every doubly stochastic direction
    Gs = g.standard_normal((P.shape[0], 4, 1)) + g.standard_normal((P.shape[0], 1, 4))
    assert np.abs(birkhoff_project_bwd(P, Gs)).max() < 1e-13
    # P = grad of a convex potential: J symmetric positive semidefinite
    s12 = (G1 * d2).sum(axis=(1, 2))
    s21 = (G2 * d1).sum(axis=(1, 2))
    np.testing.assert_allclose(s12, s21, atol=1e-13)
    assert ((G1 * d1).sum(axis=(1, 2)) >= -1e-14).all()


def test_bwd_mpmath_hard_cases():
    """60-digit solve of the same system (LU with the gauge beta_3 = 0) on the
    matrices of a large-magnitude batch whose gradients are smallest."""
    import mpmath as mp
    A = workloads.logits_batch("normal10", 400, 43).astype(np.float64)
    G = workloads.grad_batch(400, 44).astype(np.float64)
    P = birkhoff_project(A)
    dA = birkhoff_project_bwd(P, G)
    pick = list(np.argsort(np.abs(dA).max(axis=(1, 2)))[:8]) + [0, 1, 2]
    for b in pick:
        with mp.workdps(60):
            n = 4
            Pm = [[mp.mpf(float(v)) for v in row] for row in P[b]]
            Gm = [[mp.mpf(float(v)) for v in row] for row in G[b]]
            M = mp.matrix(2 * n - 1, 2 * n - 1)
            r = mp.matrix(2 * n - 1, 1)
            for i in range(n):
                M[i, i] = sum(Pm[i])
                r[i] = sum(Pm[i][j] * Gm[i][j] for j in range(n))
                for j in range(n - 1):
                    M[i, n + j] = Pm[i][j]
                    M[n + j, i] = Pm[i][j]
            for j in range(n - 1):
                M[n + j, n + j] = sum(Pm[i][j] for i in range(n))
                r[n + j] = sum(Pm[i][j] * Gm[i][j] for i in range(n))
            s = mp.lu_solve(M, r)
            al = [s[i] for i in range(n)]
            be = [s[n + j] for j in range(n - 1)] + [mp.mpf(0)]
            ref = np.array([[float(Pm[i][j] * (Gm[i][j] - al[i] - be[j])) for j in range(n)]
                            for i in range(n)])
        scale = np.abs(ref).max()
        assert np.abs(dA[b] - ref).max() <= 1e-9 * scale + 1e-20, b


def test_bwd_unrolled_sinkhorn_autograd():
    """Autograd (torch, CPU, float64) through 300 unrolled Sinkhorn sweeps --
    the memory-heavy route the summary's section 1 item 2 describes --
    agrees with the implicit gradient once Sinkhorn has converged."""
    torch = pytest.importorskip("torch")
    A = workloads.logits_batch("normal1", 64, 45).astype(np.float64)
    G = workloads.grad_batch(64, 46).astype(np.float64)
    At = torch.tensor(A, requires_grad=True)
    P = torch.exp(At - At.max(dim=2, keepdim=True).values)
    for _ in range(300):
        P = P / P.sum(dim=2, keepdim=True)
        P = P / P.sum(dim=1, keepdim=True)
    (P * torch.tensor(G)).sum().backward()
    want = birkhoff_project_bwd(birkhoff_project(A), G)
    np.testing.assert_allclose(At.grad.numpy(), want, atol=1e-10)


def test_golden_closed_forms():
    """Hand-derived exact values (tests/golden/closed_forms.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")
    with open(path) as fh:
        data = json.load(fh)
    for case in data["cases"]:
        want = np.array(case["P_num"], dtype=np.float64) / case["P_den"]
        np.testing.assert_allclose(birkhoff_project(np.array(case["A"])), want,
                                   atol=1e-14, err_msg=case["name"])
    for case in data["grad_cases"]:
        P = birkhoff_project(np.array(case["A"]))
        want = np.array(case["dA_num"], dtype=np.float64) / case["dA_den"]
        np.testing.assert_allclose(birkhoff_project_bwd(P, np.array(case["G"], dtype=np.float64)),
                                   want, atol=1e-14, err_msg=case["name"])
