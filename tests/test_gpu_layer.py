"""GPU parity of the full mHC layer step (forward and backward) against the
float64 oracle (oracle/layer.py).

Bars (elementwise, per tensor):
  rms                          |d| <= 1e-5 + 1e-5 |ref|
  logits                       |d| <= 1e-5 |ref| + 4 u sqrt(K) S2, u = 2^-24,
                               K = 4C, S2 = ||x_t o W_m||_2 / r_t: a logit is
                               a K-term fp32 sum of exact bf16 x bf16 products,
                               and its rounding grows with the terms, not with
                               the result (which can be near zero)
  H_pre, H_post                |d| <= 1e-6 + 1e-5 |ref| + H (1 - H) * (the
                               logit bar): the sigmoid's slope is H (1 - H)
  H_res                        |d| <= 1e-5 (the projection bar), against the
                               oracle's projection of the kernel's own logits
                               (the logits themselves are held to their bar)
  bf16 outputs u, x_out,       |d| <= 2^-8 |ref| + k * S, S = sum of |terms|
  grad_f, grad_x               of the output element (k = 1e-5 forward,
                               2e-4 backward: the backward carries the
                               projection gradient's 1e-4 relative bar)
  grad_logits                  |d| <= 1e-4 max|ref_t| + 1e-5 max|dH_t| per token
  grad_W                       |d| <= 2e-4 sum_t |dl_t / r_t| |x_t| + 1e-6
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import birkhoff_project
from oracle.layer import layer_bwd as o_layer_bwd
from oracle.layer import layer_fwd as o_layer_fwd

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _small_case(T, C, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    D = 4 * C
    # weight scale chosen so the residual logits have about the spread they
    # have in the 65536 x 4 x 7168 workload (0.02 * sqrt(28672) ~ 3.4)
    x = _bf16(g.standard_normal((T, 4, C)))
    Wt = _bf16(g.standard_normal((24, D)) * 3.4 / np.sqrt(D))
    f = _bf16(g.standard_normal((T, C)))
    dxo = _bf16(g.standard_normal((T, 4, C)))
    du = _bf16(g.standard_normal((T, C)))
    return x, Wt, f, dxo, du


def logit_bar(x64, W64, of):
    """Rounding bar of the logits: 4 u sqrt(K) ||x_t o W_m||_2 / r_t (u = 2^-24,
    K = 4C terms), about four standard deviations of the error of a K-term
    fp32 sum whose partial sums wander like a random walk."""
    T = x64.shape[0]
    xf = x64.reshape(T, -1)
    K = xf.shape[1]
    S2 = np.sqrt((xf * xf) @ (W64 * W64).T) / of["rms"][:, None]
    return 4.0 * 2.0 ** -24 * np.sqrt(K) * S2


def check_layer(bp, x, Wt, f, dxo, du, ref_f=None, ref_b=None, label=""):
    dev = torch.device("cuda")
    xg, Wg, fg, dxog, dug = (t.to(dev) for t in (x, Wt, f, dxo, du))
    fw = bp.layer_fwd(xg, Wg, fg)
    bw = bp.layer_bwd(xg, Wg, fg, fw, dxog, dug)
    torch.cuda.synchronize()
    x64, W64, f64, dxo64, du64 = (_f64(t) for t in (x, Wt, f, dxo, du))
    of = o_layer_fwd(x64, W64, f64) if ref_f is None else ref_f
    ob = o_layer_bwd(x64, W64, f64, dxo64, du64, fwd=of) if ref_b is None else ref_b
    g = {k: v.cpu().numpy().astype(np.float64) if v.dtype == torch.float32 else _f64(v)
         for k, v in {**fw, **bw}.items()}

    def close(name, got, want, atol, rtol=0.0):
        err = np.abs(got - want)
        bound = atol + rtol * np.abs(want)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert (err <= bound).all(), f"{label} {name}: {err[worst]:.3e} > {np.broadcast_to(bound, err.shape)[worst]:.3e} at {worst}"

    close("rms", g["rms"], of["rms"], 1e-5, 1e-5)
    bl = logit_bar(x64, W64, of)
    close("logits", g["logits"], of["logits"], bl, 1e-5)
    for k, cols in (("H_pre", slice(0, 4)), ("H_post", slice(4, 8))):
        H = of[k]
        close(k, g[k], H, 1e-6 + H * (1 - H) * bl[:, cols], 1e-5)
    close("H_res", g["H_res"], birkhoff_project(g["logits"][:, 8:].reshape(-1, 4, 4)), 1e-5)
    Hp, Ho, Hr = of["H_pre"], of["H_post"], of["H_res"]
    S_u = np.einsum("tj,tjc->tc", Hp, np.abs(x64))
    close("u", g["u"], of["u"], 2.0 ** -8 * np.abs(of["u"]) + 1e-5 * S_u + 1e-6)
    S_xo = Ho[:, :, None] * np.abs(f64)[:, None, :] + np.einsum("tij,tjc->tic", Hr, np.abs(x64))
    close("x_out", g["x_out"], of["x_out"], 2.0 ** -8 * np.abs(of["x_out"]) + 1e-5 * S_xo + 1e-6)
    S_df = np.einsum("ti,tic->tc", Ho, np.abs(dxo64))
    close("grad_f", g["grad_f"], ob["df"], 2.0 ** -8 * np.abs(ob["df"]) + 2e-4 * S_df + 1e-6)
    # grad_logits: the projection-gradient bar, scaled per token
    dH = np.concatenate([np.einsum("tc,tjc->tj", du64, x64), np.einsum("tic,tc->ti", dxo64, f64),
                         np.einsum("tic,tjc->tij", dxo64, x64).reshape(len(x64), 16)], axis=1)
    bound_l = 1e-4 * np.abs(ob["dlogits"]).max(axis=1, keepdims=True) + 1e-5 * np.abs(dH).max(axis=1, keepdims=True)
    close("grad_logits", g["grad_logits"], ob["dlogits"], bound_l)
    # grad_x
    T, n, C = x64.shape
    r = of["rms"]
    dl = ob["dlogits"]
    S_dxn = (np.abs(dl) @ np.abs(W64)).reshape(T, n, C) / r[:, None, None]
    s_coef = (dl * of["logits"]).sum(axis=1) / (n * C)
    S_dx = (np.einsum("tij,tic->tjc", Hr, np.abs(dxo64)) + Hp[:, :, None] * np.abs(du64)[:, None, :]
            + S_dxn + np.abs(x64) * np.abs(s_coef)[:, None, None] / (r ** 2)[:, None, None])
    close("grad_x", g["grad_x"], ob["dx"], 2.0 ** -8 * np.abs(ob["dx"]) + 2e-4 * S_dx + 1e-6)
    # grad_W
    xn_abs = np.abs(x64.reshape(T, -1)) / r[:, None]
    S_W = np.abs(dl).T @ xn_abs
    close("grad_W", g["grad_W"], ob["dW"], 2e-4 * S_W + 1e-6)
    return fw, bw


@pytest.mark.parametrize("T,C", [(1, 64), (37, 64), (64, 128), (130, 192)])
def test_layer_small(gpu_lib, T, C):
    print(f"layer parity T={T} C={C}", flush=True)
    check_layer(gpu_lib, *_small_case(T, C, 1000 + T), label=f"T={T} C={C}")


def test_layer_repeatable(gpu_lib):
    """Same inputs twice give bit-identical outputs (no atomics, fixed-order
    reductions)."""
    x, Wt, f, dxo, du = (t.cuda() for t in _small_case(100, 128, 77))
    a = gpu_lib.layer_fwd(x, Wt, f)
    ga = gpu_lib.layer_bwd(x, Wt, f, a, dxo, du)
    b = gpu_lib.layer_fwd(x, Wt, f)
    gb = gpu_lib.layer_bwd(x, Wt, f, b, dxo, du)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    for k in ga:
        assert torch.equal(ga[k], gb[k]), k


@pytest.mark.parametrize("T", [2048, 4000])
def test_layer_grad_w_token_groups(gpu_lib, T):
    """grad_W summed over 16 token groups, as at the workload's size.  The
    backward splits the padded batch (T rounded up to 64) into at most 16
    groups of whole 128-token rounds, writes one partial per group and adds
    the partials in a fixed order.  T = 2048 gives 16 groups of 128 tokens;
    T = 4000 (padded to 4032) gives 15 groups of 256 and a last one of 192,
    whose final 32 tokens are padding.  Every output, grad_W included, is
    compared element-wise with the oracle."""
    C = 512
    print(f"layer token groups T={T} C={C}", flush=True)
    check_layer(gpu_lib, *_small_case(T, C, 3000 + T), label=f"T={T} C={C}")


def test_layer_full_size(gpu_lib):
    """T=65536, n=4, C=7168 (seed 5): the whole step at full size in the same
    launch configuration the bench times.

    * Every token's rms, logits, H_pre, H_post, H_res and grad_logits, and
      every entry of grad_W (the sum over all 65536 tokens in 16 token
      groups), against the oracle, which runs over the batch in chunks of
      2048 tokens without its stream-width outputs.
    * u, x_out, grad_f and grad_x (the stream-width outputs) on 48 sampled
      tokens against the full oracle."""
    T, C = W.CONFIG5_SHAPE["T"], W.CONFIG5_SHAPE["C"]
    inp = W.layer_inputs(T, C, seed=5)
    x, Wt, f, dxo, du = inp["x"], inp["W"], inp["f"], inp["dx_out"], inp["du"]
    fw = gpu_lib.layer_fwd(x, Wt, f)
    bw = gpu_lib.layer_bwd(x, Wt, f, fw, dxo, du)
    torch.cuda.synchronize()
    W64 = _f64(Wt)
    D = 4 * C

    failures = []

    def close(name, got, want, bound):
        err = np.abs(got - want)
        bad = err > bound
        if bad.any():
            worst = np.unravel_index(np.argmax(err - bound), err.shape)
            failures.append(f"{name}: {int(bad.sum())} over the bar, worst {err[worst]:.3e} > "
                            f"{np.broadcast_to(bound, err.shape)[worst]:.3e} at {worst}")

    # 1. the per-token maps and grad_logits of every token, and grad_W
    dW = np.zeros((24, D))
    S_W = np.zeros((24, D))
    chunk = 2048
    for t0 in range(0, T, chunk):
        sl = slice(t0, t0 + chunk)
        xs, fs, dxos, dus = (_f64(t[sl]) for t in (x, f, dxo, du))
        of = o_layer_fwd(xs, W64, fs, streams=False)
        ob = o_layer_bwd(xs, W64, fs, dxos, dus, fwd=of, streams=False)
        got = {k: fw[k][sl].cpu().numpy().astype(np.float64)
               for k in ("rms", "logits", "H_pre", "H_post", "H_res")}
        close(f"rms[{t0}:]", got["rms"], of["rms"], 1e-5 + 1e-5 * np.abs(of["rms"]))
        bl = logit_bar(xs, W64, of)
        close(f"logits[{t0}:]", got["logits"], of["logits"], bl + 1e-5 * np.abs(of["logits"]))
        for k, cols in (("H_pre", slice(0, 4)), ("H_post", slice(4, 8))):
            H = of[k]
            close(f"{k}[{t0}:]", got[k], H, 1e-6 + 1e-5 * H + H * (1 - H) * bl[:, cols])
        close(f"H_res[{t0}:]", got["H_res"],
              birkhoff_project(got["logits"][:, 8:].reshape(-1, 4, 4)), 1e-5)
        dH = np.concatenate([np.einsum("tc,tjc->tj", dus, xs), np.einsum("tic,tc->ti", dxos, fs),
                             np.einsum("tic,tjc->tij", dxos, xs).reshape(len(xs), 16)], axis=1)
        bound = (1e-4 * np.abs(ob["dlogits"]).max(axis=1, keepdims=True)
                 + 1e-5 * np.abs(dH).max(axis=1, keepdims=True))
        close(f"grad_logits[{t0}:]", bw["grad_logits"][sl].cpu().numpy().astype(np.float64),
              ob["dlogits"], bound)
        dW += ob["dW"]
        S_W += np.abs(ob["dlogits"]).T @ (np.abs(xs.reshape(len(xs), D)) / of["rms"][:, None])
    close("grad_W", bw["grad_W"].cpu().numpy().astype(np.float64), dW, 2e-4 * S_W + 1e-6)

    # 2. the stream-width outputs on a sample of tokens
    g = np.random.Generator(np.random.PCG64(55))
    idx = torch.from_numpy(np.sort(g.choice(T, 48, replace=False))).cuda()
    xs, fs, dxos, dus = (_f64(t[idx]) for t in (x, f, dxo, du))
    of = o_layer_fwd(xs, W64, fs)
    ob = o_layer_bwd(xs, W64, fs, dxos, dus, fwd=of)
    u = _f64(fw["u"][idx])
    S_u = np.einsum("tj,tjc->tc", of["H_pre"], np.abs(xs))
    close("u", u, of["u"], 2.0 ** -8 * np.abs(of["u"]) + 1e-5 * S_u + 1e-6)
    xo = _f64(fw["x_out"][idx])
    S_xo = of["H_post"][:, :, None] * np.abs(fs)[:, None, :] + np.einsum("tij,tjc->tic", of["H_res"], np.abs(xs))
    close("x_out", xo, of["x_out"], 2.0 ** -8 * np.abs(of["x_out"]) + 1e-5 * S_xo + 1e-6)
    gf = _f64(bw["grad_f"][idx])
    S_df = np.einsum("ti,tic->tc", of["H_post"], np.abs(dxos))
    close("grad_f", gf, ob["df"], 2.0 ** -8 * np.abs(ob["df"]) + 2e-4 * S_df + 1e-6)
    gx = _f64(bw["grad_x"][idx])
    r = of["rms"]
    S_dxn = (np.abs(ob["dlogits"]) @ np.abs(W64)).reshape(len(xs), 4, C) / r[:, None, None]
    s_coef = (ob["dlogits"] * of["logits"]).sum(axis=1) / (4 * C)
    S_dx = (np.einsum("tij,tic->tjc", of["H_res"], np.abs(dxos)) + of["H_pre"][:, :, None] * np.abs(dus)[:, None, :]
            + S_dxn + np.abs(xs) * np.abs(s_coef)[:, None, None] / (r ** 2)[:, None, None])
    close("grad_x", gx, ob["dx"], 2.0 ** -8 * np.abs(ob["dx"]) + 2e-4 * S_dx + 1e-6)
    assert not failures, "\n".join(failures)


def test_layer_sinkhorn_solver(gpu_lib):
    """The layer forward with the Sinkhorn-Knopp solver for H_res (opts
    solver = Sinkhorn, run to tol): H_res within the projection bar of the
    oracle's projection of the kernel's own logits; the maps, rms and u
    (which does not involve H_res) bit for bit the Newton run's; x_out
    within its two bf16 roundings plus what H_res moves it (each entry of
    both H_res within 1e-5 of the projection, so at most 4 x 2e-5 max|x|)."""
    x, Wt, f, _, _ = _small_case(64, 128, 77)
    dev = torch.device("cuda")
    xg, Wg, fg = (t.to(dev) for t in (x, Wt, f))
    fn = gpu_lib.layer_fwd(xg, Wg, fg)
    fs = gpu_lib.layer_fwd(xg, Wg, fg, solver="sinkhorn", tol=1e-6)
    torch.cuda.synchronize()
    for k in ("rms", "logits", "H_pre", "H_post", "u"):
        assert torch.equal(fs[k], fn[k]), k
    logits = fs["logits"].cpu().numpy().astype(np.float64)[:, 8:].reshape(-1, 4, 4)
    assert np.abs(fs["H_res"].cpu().numpy() - birkhoff_project(logits)).max() <= 1e-5
    a, b = fs["x_out"].float(), fn["x_out"].float()
    bound = 2.0 ** -7 * b.abs() + 4 * 2e-5 * xg.float().abs().amax() + 1e-6
    assert bool(((a - b).abs() <= bound).all())
