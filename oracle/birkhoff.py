"""Float64 CPU oracle for the Birkhoff projection of mHC and its gradient.

TEST INFRASTRUCTURE ONLY.  This module is imported by tests/, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
nothing in the product package imports it, and it imports nothing from there.
It is plain and slow on purpose: every step is written the way the pages
state it, in float64, with no blocking, fusion or reordering.

What it computes
----------------
Forward.  For a real n x n matrix A (a row of residual-mixing logits per
token), K = exp(A) is entrywise positive and there is exactly one doubly
stochastic matrix of the form diag(u) K diag(v).  That matrix is the
projection P(A).  It is the fixed point of Sinkhorn-Knopp (alternately divide
every row by its sum, then every column by its sum) -- Deep Signal mHC article,
section "Implementing the constraint projection with Sinkhorn-Knopp"; forpes.ru
mHC explainer, section "mHC: bring back the guarantee" -- and the solution of
the entropy-regularised transport problem max_P <P,A> - sum P log P over the
Birkhoff polytope ("Accelerating Birkhoff projection for mHC", gist.science
summary, section 2 "Method").  Before the exponential every row is shifted by
its maximum (same summary, section 2.1, "numerical stability"); the shift does
not change P because a row scaling is absorbed into u.

The oracle runs Sinkhorn-Knopp sweeps (rows, then columns) until the largest
row or column sum error is below ``tol`` (1e-13).  Matrices that have not got
there after ``max_sweeps`` sweeps -- Sinkhorn is slow on large-magnitude
inputs, section 1 "Problem statement", item 3 of the same summary -- are
finished by Newton's method on the full two-sided dual (f, g) in float64 with
a gauge row, followed by one more Sinkhorn sweep.  This is deliberately not
the reduced three-variable dual of section 2.1.  Anything still above ``tol``
goes to a 50-digit mpmath solve.

Backward.  dL/dA = J^T G with J = dP/dA.  By the implicit function theorem on
the scaling conditions (section 2.2 "Backward pass: implicit differentiation"),
    dA = P o (G - alpha 1^T - 1 beta^T),
    [[I, P], [P^T, I]] [alpha; beta] = [(P o G) 1; (P o G)^T 1],
a singular but consistent 2n x 2n system (null vector [1; -1]); every solution
gives the same dA.  The oracle solves it as the equivalent weighted
least-squares fit (Householder QR on the full 2n-variable problem), not the
reduced (I - P^T P) form the GPU path uses.

Pins: tests/test_oracle_birkhoff.py (closed forms, invariants, 50-digit
brute force, finite differences, unrolled-Sinkhorn autograd).
"""
from __future__ import annotations

import numpy as np

SINKHORN_TOL = 1e-13
EXTREME_SPREAD = 600.0


def residual(P: np.ndarray) -> np.ndarray:
    """Largest |row sum - 1| or |column sum - 1| per matrix (float64)."""
    P = np.asarray(P, dtype=np.float64)
    r = np.abs(P.sum(axis=-1) - 1.0).max(axis=-1)
    c = np.abs(P.sum(axis=-2) - 1.0).max(axis=-1)
    return np.maximum(r, c)


def row_max_shift(A: np.ndarray) -> np.ndarray:
    """A with each row shifted so that its largest entry is 0."""
    return A - A.max(axis=-1, keepdims=True)


def sinkhorn(A, tol=SINKHORN_TOL, max_sweeps=500):
    """Sinkhorn-Knopp on K = exp(row-max-shifted A), batched over the first dim.

    One sweep divides each row by its row sum, then each column by its column
    sum.  A matrix stops as soon as its residual is below ``tol``.

    Returns (P, f, g, sweeps, converged) with P = exp(L + f_i + g_j) where L is
    the row-max-shifted A, so the caller can continue in the log domain.
    """
    A = np.asarray(A, dtype=np.float64)
    B, n, _ = A.shape
    L = row_max_shift(A)
    P = np.exp(L)
    f = np.zeros((B, n))
    g = np.zeros((B, n))
    sweeps = np.zeros(B, dtype=np.int64)
    active = np.arange(B)
    for _ in range(max_sweeps):
        if active.size == 0:
            break
        Q = P[active]
        r = Q.sum(axis=2)
        Q = Q / r[:, :, None]
        c = Q.sum(axis=1)
        Q = Q / c[:, None, :]
        P[active] = Q
        f[active] -= np.log(r)
        g[active] -= np.log(c)
        sweeps[active] += 1
        done = residual(Q) < tol
        active = active[~done]
    converged = np.ones(B, dtype=bool)
    converged[active] = False
    return P, f, g, sweeps, converged


def _dual_value(L, f, g):
    """Dual objective of the scaling problem, sum_ij exp(L+f_i+g_j) - sum f - sum g.
    Convex; its gradient is (row sums - 1, column sums - 1)."""
    P = np.exp(L + f[:, :, None] + g[:, None, :])
    return P.sum(axis=(1, 2)) - f.sum(axis=1) - g.sum(axis=1)


def newton_two_sided(L, f, g, iters=60, tol=SINKHORN_TOL, max_step=30.0):
    """Newton's method on the two-sided dual (f, g) for a batch, float64.

    Hessian [[diag r, P], [P^T, diag c]] is singular along (1, -1); the gauge
    row sum(f) - sum(g) = 0 is appended (bordered system).  Armijo
    backtracking on the dual objective; near the solution, where the objective
    no longer changes in float64, a step is also accepted if it halves the
    gradient.  Returns updated (f, g).
    """
    B, n, _ = L.shape
    f = f.copy()
    g = g.copy()
    e = np.concatenate([np.ones(n), -np.ones(n)])
    for _ in range(iters):
        P = np.exp(L + f[:, :, None] + g[:, None, :])
        r = P.sum(axis=2)
        c = P.sum(axis=1)
        grad = np.concatenate([r - 1.0, c - 1.0], axis=1)
        gnorm = np.abs(grad).max(axis=1)
        act = gnorm >= tol * 0.25
        if not act.any():
            break
        idx = np.nonzero(act)[0]
        Pa = P[idx]
        m = idx.size
        H = np.zeros((m, 2 * n + 1, 2 * n + 1))
        H[:, :n, :n] = r[idx][:, :, None] * np.eye(n)
        H[:, n:2 * n, n:2 * n] = c[idx][:, :, None] * np.eye(n)
        H[:, :n, n:2 * n] = Pa
        H[:, n:2 * n, :n] = np.swapaxes(Pa, 1, 2)
        H[:, :2 * n, 2 * n] = e
        H[:, 2 * n, :2 * n] = e
        rhs = np.concatenate([-grad[idx], np.zeros((m, 1))], axis=1)
        step = np.linalg.solve(H, rhs[:, :, None])[:, :2 * n, 0]
        # Near-decomposable matrices make the system nearly singular and the
        # Newton step enormous along the weakly coupled direction; the line
        # search starts from a step no longer than max_step instead.
        smax = np.abs(step).max(axis=1)
        step = step * np.minimum(1.0, max_step / np.maximum(smax, 1e-300))[:, None]
        df, dg = step[:, :n], step[:, n:]
        fa, ga, La = f[idx], g[idx], L[idx]
        phi0 = _dual_value(La, fa, ga)
        slope = (grad[idx] * step).sum(axis=1)
        t = np.ones(m)
        accepted = np.zeros(m, dtype=bool)
        for _ls in range(60):
            todo = ~accepted
            if not todo.any():
                break
            fn = fa + t[:, None] * df
            gn = ga + t[:, None] * dg
            phi = _dual_value(La, fn, gn)
            Pn = np.exp(La + fn[:, :, None] + gn[:, None, :])
            gn_norm = np.maximum(np.abs(Pn.sum(axis=2) - 1.0).max(axis=1),
                                 np.abs(Pn.sum(axis=1) - 1.0).max(axis=1))
            ok = (phi <= phi0 + 1e-4 * t * slope) | (gn_norm <= 0.5 * gnorm[idx])
            newly = todo & ok
            accepted |= newly
            t = np.where(todo & ~ok, 0.5 * t, t)
        # a matrix whose line search found no acceptable step keeps its point
        t = np.where(accepted, t, 0.0)
        f[idx] = fa + t[:, None] * df
        g[idx] = ga + t[:, None] * dg
    return f, g


def _mp_project_one(A_row, dps=50, tol_digits=40):
    """One matrix in mpmath at ``dps`` digits: Sinkhorn sweeps for a start,
    then Newton on the two-sided dual with the gauge g[-1] = 0 (solve the
    2n-1 independent scaling equations).  Returns float64 P."""
    import mpmath as mp
    n = len(A_row)
    with mp.workdps(dps):
        L = [[mp.mpf(float(A_row[i][j])) for j in range(n)] for i in range(n)]
        for i in range(n):
            mx = max(L[i])
            L[i] = [v - mx for v in L[i]]
        f = [mp.mpf(0)] * n
        g = [mp.mpf(0)] * n

        def mat(f, g):
            return [[mp.e ** (L[i][j] + f[i] + g[j]) for j in range(n)] for i in range(n)]

        for _ in range(200):
            P = mat(f, g)
            for i in range(n):
                f[i] -= mp.log(sum(P[i]))
            P = mat(f, g)
            for j in range(n):
                g[j] -= mp.log(sum(P[i][j] for i in range(n)))
        shift = g[n - 1]
        g = [v - shift for v in g]
        f = [v + shift for v in f]
        eps = mp.mpf(10) ** (-tol_digits)
        for _ in range(200):
            P = mat(f, g)
            r = [sum(P[i]) - 1 for i in range(n)]
            c = [sum(P[i][j] for i in range(n)) - 1 for j in range(n)]
            res = max(abs(v) for v in r + c)
            if res < eps:
                break
            # unknowns f_0..f_{n-1}, g_0..g_{n-2}; equations r_0..r_{n-1}, c_0..c_{n-2}
            m = 2 * n - 1
            J = mp.matrix(m, m)
            F = mp.matrix(m, 1)
            for i in range(n):
                F[i] = r[i]
                J[i, i] = r[i] + 1
                for j in range(n - 1):
                    J[i, n + j] = P[i][j]
            for j in range(n - 1):
                F[n + j] = c[j]
                J[n + j, n + j] = c[j] + 1
                for i in range(n):
                    J[n + j, i] = P[i][j]
            d = mp.lu_solve(J, -F)
            t = mp.mpf(1)
            for _ls in range(60):
                fn = [f[i] + t * d[i] for i in range(n)]
                gn = [g[j] + t * d[n + j] for j in range(n - 1)] + [g[n - 1]]
                Pn = mat(fn, gn)
                rn = max([abs(sum(Pn[i]) - 1) for i in range(n)]
                         + [abs(sum(Pn[i][j] for i in range(n)) - 1) for j in range(n)])
                if rn < res:
                    break
                t /= 2
            f, g = fn, gn
        P = mat(f, g)
        return np.array([[float(P[i][j]) for j in range(n)] for i in range(n)])


def birkhoff_project(A, tol=SINKHORN_TOL, max_sweeps=100, newton_iters=60,
                     return_info=False):
    """The projection P(A) of a batch [B,n,n] onto the doubly stochastic
    matrices, float64, residual < tol for every matrix.

    Steps: exp after the row max-shift; Sinkhorn sweeps; for the unconverged,
    Newton on the two-sided dual then one Sinkhorn sweep; for any still above
    tol, a 50-digit mpmath solve.
    """
    A = np.asarray(A, dtype=np.float64)
    squeeze = A.ndim == 2
    if squeeze:
        A = A[None]
    if not np.all(np.isfinite(A)):
        raise ValueError("oracle: logits must be finite")
    # a row spread beyond ~700 underflows float64 exp to exact zeros, which
    # can leave no representable scaling: such matrices go to mpmath directly
    extreme = (A.max(axis=-1) - A.min(axis=-1)).max(axis=-1) > EXTREME_SPREAD
    P, f, g, sweeps, conv = sinkhorn(np.where(extreme[:, None, None], 0.0, A), tol=tol,
                                     max_sweeps=max_sweeps)
    conv &= ~extreme
    polished = ~conv & ~extreme
    mp_used = np.zeros(A.shape[0], dtype=bool)
    if polished.any():
        idx = np.nonzero(polished)[0]
        L = row_max_shift(A[idx])
        fi, gi = newton_two_sided(L, f[idx], g[idx], iters=newton_iters, tol=tol)
        Q = np.exp(L + fi[:, :, None] + gi[:, None, :])
        Q = Q / Q.sum(axis=2, keepdims=True)
        Q = Q / Q.sum(axis=1, keepdims=True)
        P[idx] = Q
    bad = np.nonzero((residual(P) >= tol) | extreme)[0]
    for b in bad:
        P[b] = _mp_project_one(A[b])
        mp_used[b] = True
    if np.any(residual(P) >= tol):
        raise RuntimeError("oracle: projection failed to reach the tolerance")
    P = P[0] if squeeze else P
    if return_info:
        return P, dict(sweeps=sweeps, polished=polished, mp=mp_used)
    return P


def birkhoff_project_bwd(P, G, chunk=65536):
    """dL/dA for the projection, given P = P(A) and G = dL/dP (float64).

    The implicit-differentiation system of section 2.2 of the summary,
        [[diag r, P], [P^T, diag c]] [alpha; beta] = [(P o G) 1; (P o G)^T 1],
    is the normal-equation form of a weighted least-squares fit of G by a
    row effect plus a column effect,
        min over (alpha, beta) of  sum_ij P_ij (G_ij - alpha_i - beta_j)^2,
    and dA = P o (G - alpha 1^T - 1 beta^T) is P times that fit's residual.
    The oracle solves the fit itself, not its normal equations: the n*n x
    (2n-1) matrix with rows sqrt(P_ij) (e_i + e_{n+j}) (gauge beta_{n-1} = 0,
    which fixes the one-dimensional null space alpha + c, beta - c) is
    factored by Householder QR and the residual is formed as (I - Q Q^T) y.
    This stays accurate when P is close to a permutation, where the normal
    equations become nearly singular.
    """
    P = np.asarray(P, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    squeeze = P.ndim == 2
    if squeeze:
        P, G = P[None], G[None]
    B, n, _ = P.shape
    out = np.empty_like(P)
    # design matrix of the fit, unweighted: row (i, j) picks alpha_i and beta_j
    design = np.zeros((n * n, 2 * n - 1))
    for i in range(n):
        for j in range(n):
            design[i * n + j, i] = 1.0
            if j < n - 1:
                design[i * n + j, n + j] = 1.0
    for s in range(0, B, chunk):
        Pc, Gc = P[s:s + chunk], G[s:s + chunk]
        w = np.sqrt(Pc.reshape(-1, n * n))
        Xw = w[:, :, None] * design[None]
        y = w * Gc.reshape(-1, n * n)
        Q, _ = np.linalg.qr(Xw)
        resid = y - np.einsum("bkm,bm->bk", Q, np.einsum("bkm,bk->bm", Q, y))
        out[s:s + chunk] = (w * resid).reshape(-1, n, n)
    return out[0] if squeeze else out


def sinkhorn_fixed(A, sweeps):
    """Exactly ``sweeps`` Sinkhorn-Knopp sweeps (rows then columns) on
    exp(row-max-shifted A), the fixed-iteration practice that section 1 of
    the summary describes ("e.g. 20 iterations").  float64."""
    A = np.asarray(A, dtype=np.float64)
    P = np.exp(row_max_shift(A))
    for _ in range(sweeps):
        P = P / P.sum(axis=-1, keepdims=True)
        P = P / P.sum(axis=-2, keepdims=True)
    return P
