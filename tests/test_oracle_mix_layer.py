"""Pins for the stream-mix and full-layer oracles (oracle/mix.py,
oracle/layer.py).  No GPU."""
import numpy as np
import pytest

import workloads
from oracle import birkhoff_project
from oracle.layer import layer_bwd, layer_fwd
from oracle.mix import stream_mix, stream_mix_bwd


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_mix_brute_force_loops():
    g = _rng(1)
    H = g.standard_normal((3, 4, 4))
    x = g.standard_normal((3, 4, 5))
    out = stream_mix(H, x)
    for t in range(3):
        for i in range(4):
            for c in range(5):
                s = 0.0
                for j in range(4):
                    s += H[t, i, j] * x[t, j, c]
                assert abs(out[t, i, c] - s) < 1e-14


def test_mix_identity_and_permutation():
    x = _rng(2).standard_normal((5, 4, 33))
    np.testing.assert_array_equal(stream_mix(np.broadcast_to(np.eye(4), (5, 4, 4)), x), x)
    perm = np.eye(4)[[2, 0, 3, 1]]
    np.testing.assert_array_equal(stream_mix(np.broadcast_to(perm, (5, 4, 4)), x), x[:, [2, 0, 3, 1]])


def test_mix_mean_preservation():
    """Doubly stochastic H keeps the sum over streams (neo-ai mHC summary:
    feature means are preserved)."""
    A = workloads.logits_batch("normal2", 50, 3)
    H = birkhoff_project(A)
    x = _rng(4).standard_normal((50, 4, 64))
    np.testing.assert_allclose(stream_mix(H, x).sum(axis=1), x.sum(axis=1), atol=1e-12)


def test_mix_bwd_adjoint_identities():
    """out is bilinear in (H, x): <dout, out> = <dx, x> = <dH, H>."""
    g = _rng(5)
    H = g.standard_normal((7, 4, 4))
    x = g.standard_normal((7, 4, 19))
    dout = g.standard_normal((7, 4, 19))
    dx, dH = stream_mix_bwd(H, x, dout)
    s = (dout * stream_mix(H, x)).sum(axis=(1, 2))
    np.testing.assert_allclose((dx * x).sum(axis=(1, 2)), s, atol=1e-12)
    np.testing.assert_allclose((dH * H).sum(axis=(1, 2)), s, atol=1e-12)


def test_mix_bwd_brute_force_loops():
    g = _rng(6)
    H = g.standard_normal((2, 4, 4))
    x = g.standard_normal((2, 4, 3))
    dout = g.standard_normal((2, 4, 3))
    dx, dH = stream_mix_bwd(H, x, dout)
    for t in range(2):
        for j in range(4):
            for c in range(3):
                s = sum(H[t, i, j] * dout[t, i, c] for i in range(4))
                assert abs(dx[t, j, c] - s) < 1e-14
        for i in range(4):
            for j in range(4):
                s = sum(dout[t, i, c] * x[t, j, c] for c in range(3))
                assert abs(dH[t, i, j] - s) < 1e-14


# ---------------------------------------------------------------------------
# layer
# ---------------------------------------------------------------------------

def _layer_case(T=3, n=4, C=5, seed=7, wscale=0.3):
    g = _rng(seed)
    x = g.standard_normal((T, n, C))
    W = g.standard_normal((n * n + 2 * n, n * C)) * wscale
    f = g.standard_normal((T, C))
    dx_out = g.standard_normal((T, n, C))
    du = g.standard_normal((T, C))
    return x, W, f, dx_out, du


def test_layer_fwd_structure():
    x, W, f, _, _ = _layer_case()
    out = layer_fwd(x, W, f)
    T, n, C = x.shape
    xf = x.reshape(T, -1)
    # the normalised stream has mean square 1 - eps / r^2
    xn = xf / out["rms"][:, None]
    np.testing.assert_allclose((xn ** 2).mean(axis=1), 1 - 1e-6 / out["rms"] ** 2, atol=1e-14)
    assert ((out["H_pre"] > 0) & (out["H_pre"] < 1)).all()
    assert ((out["H_post"] > 0) & (out["H_post"] < 1)).all()
    from oracle import residual
    assert residual(out["H_res"]).max() < 1e-13
    # u and x_out from explicit loops
    for t in range(T):
        for c in range(C):
            u = sum(out["H_pre"][t, j] * x[t, j, c] for j in range(n))
            assert abs(out["u"][t, c] - u) < 1e-13
            for i in range(n):
                xo = out["H_post"][t, i] * f[t, c] + sum(out["H_res"][t, i, j] * x[t, j, c] for j in range(n))
                assert abs(out["x_out"][t, i, c] - xo) < 1e-13


def test_layer_identity_residual_limit():
    """Degenerate map W = 0: every logit is 0, so H_pre = H_post = 1/2 and
    H_res = J/4 (rank-one kernel), and u is half the stream sum."""
    x, W, f, _, _ = _layer_case()
    out = layer_fwd(x, np.zeros_like(W), f)
    np.testing.assert_allclose(out["H_pre"], 0.5)
    np.testing.assert_allclose(out["H_res"], 0.25, atol=1e-14)
    np.testing.assert_allclose(out["u"], 0.5 * x.sum(axis=1), atol=1e-13)


def test_layer_logits_scale_invariant():
    """With eps = 0 the RMS-normalised stream, hence every logit and map, is
    unchanged when x is scaled; u scales with x.  A logit formed from the raw
    stream, or normalised over one stream instead of all n C values, fails
    this."""
    x, W, f, _, _ = _layer_case(seed=12)
    a = layer_fwd(x, W, f, eps=0.0)
    b = layer_fwd(3.0 * x, W, f, eps=0.0)
    for k in ("logits", "H_pre", "H_post", "H_res"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-13, atol=1e-14, err_msg=k)
    np.testing.assert_allclose(b["u"], 3.0 * a["u"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b["rms"], 3.0 * a["rms"], rtol=1e-14)


def _one_hot_res(a):
    """Projection of the 4 x 4 logit matrix with the single nonzero entry a at
    (i, j): swapping any two other rows or columns leaves the kernel
    exp(L) unchanged, so P is p at (i, j), (1 - p)/3 elsewhere in row i and
    column j, and (2 + p)/9 everywhere else, and the scaling condition
    P_ij P_kl / (P_il P_kj) = e^a for k != i, l != j gives
    p (2 + p) = e^a (1 - p)^2, solved here for the root in (0, 1)."""
    e = np.exp(a)
    qa, qb, qc = 1.0 - e, 2.0 + 2.0 * e, -e
    with np.errstate(divide="ignore", invalid="ignore"):
        root = (-qb + np.sqrt(qb * qb - 4.0 * qa * qc)) / (2.0 * qa)
    return np.where(np.abs(qa) < 1e-12, 0.25, root)


@pytest.mark.parametrize("m", [0, 5, 8, 8 + 4 * 1 + 2, 8 + 4 * 3 + 0])
def test_layer_one_hot_map(m):
    """W with a single 1 at row m, column k: logit m is x_flat[k] / r and every
    other logit 0.  So H_pre and H_post are 1/2 except sigmoid(x_k / r) at
    entry m (pre rows 0:4, post rows 4:8), and for a residual row
    m = 8 + 4 i + j, H_res is the closed-form projection of a matrix with one
    nonzero entry at (i, j).  Catches a transposed W, a misplaced block or a
    misordered residual matrix."""
    x, _, f, _, _ = _layer_case(T=6, C=5, seed=13)
    T, n, C = x.shape
    k = 7
    W = np.zeros((n * n + 2 * n, n * C))
    W[m, k] = 1.0
    out = layer_fwd(x, W, f)
    xf = x.reshape(T, -1)
    lm = xf[:, k] / out["rms"]
    expect = np.zeros((T, n * n + 2 * n))
    expect[:, m] = lm
    np.testing.assert_allclose(out["logits"], expect, atol=1e-15, rtol=1e-14)
    sig = 1.0 / (1.0 + np.exp(-lm))
    pre = np.full((T, n), 0.5)
    post = np.full((T, n), 0.5)
    if m < n:
        pre[:, m] = sig
    elif m < 2 * n:
        post[:, m - n] = sig
    np.testing.assert_allclose(out["H_pre"], pre, atol=1e-15)
    np.testing.assert_allclose(out["H_post"], post, atol=1e-15)
    if m >= 2 * n:
        i, j = divmod(m - 2 * n, n)
        p = _one_hot_res(lm)
        H = np.empty((T, n, n))
        H[:] = ((2.0 + p) / 9.0)[:, None, None]
        H[:, i, :] = ((1.0 - p) / 3.0)[:, None]
        H[:, :, j] = ((1.0 - p) / 3.0)[:, None]
        H[:, i, j] = p
        np.testing.assert_allclose(out["H_res"], H, atol=1e-12)
    else:
        np.testing.assert_allclose(out["H_res"], 0.25, atol=1e-14)


def _loss(x, W, f, dx_out, du):
    out = layer_fwd(x, W, f)
    return (out["x_out"] * dx_out).sum() + (out["u"] * du).sum()


@pytest.mark.parametrize("seed", [8, 9])
def test_layer_bwd_finite_differences(seed):
    """Central differences (h = 1e-6) of L = <dx_out, x_out> + <du, u> with
    respect to every entry of x, W and f on a tiny case."""
    x, W, f, dx_out, du = _layer_case(T=2, C=3, seed=seed)
    g = layer_bwd(x, W, f, dx_out, du)
    h = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("W", W, g["dW"]), ("f", f, g["df"])):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap = arr.copy()
            am = arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = dict(x=x, W=W, f=f)
            args_m = dict(x=x, W=W, f=f)
            args_p[name] = ap
            args_m[name] = am
            fd[idx] = (_loss(args_p["x"], args_p["W"], args_p["f"], dx_out, du)
                       - _loss(args_m["x"], args_m["W"], args_m["f"], dx_out, du)) / (2 * h)
        np.testing.assert_allclose(grad, fd, atol=2e-7, rtol=1e-6, err_msg=name)


def test_layer_bwd_torch_autograd():
    """Torch float64 autograd of the same step, with the projection taken as
    800 unrolled Sinkhorn sweeps on moderate logits (converged to 1e-15)."""
    torch = pytest.importorskip("torch")
    x, W, f, dx_out, du = _layer_case(T=4, C=6, seed=10, wscale=0.15)
    tx, tW, tf = (torch.tensor(a, requires_grad=True) for a in (x, W, f))
    T, n, C = x.shape
    xf = tx.reshape(T, -1)
    r = torch.sqrt((xf * xf).mean(dim=1) + 1e-6)
    l = (xf / r[:, None]) @ tW.T
    hp = torch.sigmoid(l[:, :n])
    ho = torch.sigmoid(l[:, n:2 * n])
    Lr = l[:, 2 * n:].reshape(T, n, n)
    P = torch.exp(Lr - Lr.max(dim=2, keepdim=True).values)
    for _ in range(800):
        P = P / P.sum(dim=2, keepdim=True)
        P = P / P.sum(dim=1, keepdim=True)
    u = torch.einsum("tj,tjc->tc", hp, tx)
    xo = ho[:, :, None] * tf[:, None, :] + torch.einsum("tij,tjc->tic", P, tx)
    loss = (xo * torch.tensor(dx_out)).sum() + (u * torch.tensor(du)).sum()
    loss.backward()
    g = layer_bwd(x, W, f, dx_out, du)
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(g["dW"], tW.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(g["df"], tf.grad.numpy(), atol=1e-10)


def test_layer_without_streams_matches():
    """layer_fwd / layer_bwd with streams=False return the same maps,
    logits gradient and dW as the full computation (they only skip u, x_out,
    dx and df)."""
    from oracle.layer import layer_bwd, layer_fwd
    g = np.random.Generator(np.random.PCG64(91))
    T, C = 9, 16
    x = g.standard_normal((T, 4, C))
    W = g.standard_normal((24, 4 * C)) * 0.3
    f = g.standard_normal((T, C))
    dxo = g.standard_normal((T, 4, C))
    du = g.standard_normal((T, C))
    a = layer_fwd(x, W, f)
    b = layer_fwd(x, W, f, streams=False)
    assert set(b) == {"rms", "logits", "H_pre", "H_post", "H_res"}
    for k in b:
        np.testing.assert_array_equal(a[k], b[k])
    ga = layer_bwd(x, W, f, dxo, du, fwd=a)
    gb = layer_bwd(x, W, f, dxo, du, fwd=b, streams=False)
    assert set(gb) == {"dW", "dlogits"}
    for k in gb:
        np.testing.assert_array_equal(ga[k], gb[k])
