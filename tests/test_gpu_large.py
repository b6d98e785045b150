"""Sizes past 2^31 elements: every index in the kernels is 64-bit, so batches
whose element offsets exceed the int32 range must come out like small ones.
Inputs are drawn on the device (seeded torch generator); sampled matrices and
tokens -- the last ones, ones around the 2^31-element boundary and a seeded
random set -- are checked against the float64 oracle, and nothing past the
batch may be written.  Needs about 45 GB of device memory."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import birkhoff_project, birkhoff_project_bwd, stream_mix

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _randn(shape, gen, scale, chunk=1 << 24):
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk):
        r1 = min(shape[0], r0 + chunk)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device="cuda") * scale
    return out


def test_projection_past_int32_offsets(gpu_lib):
    B = (1 << 27) + 37          # 16 B > 2^31 floats
    print(f"large projection B={B}", flush=True)
    gen = W._torch_gen(2701, "cuda")
    A = _randn((B, 4, 4), gen, 10.0)
    Pfull = torch.full((B + 64, 4, 4), SENTINEL, device="cuda")
    P = Pfull[:B]
    _, it = gpu_lib.birkhoff_fwd(A, out=P, return_iters=True)
    G = _randn((B, 4, 4), gen, 1.0)
    dfull = torch.full((B + 64, 4, 4), SENTINEL, device="cuda")
    gpu_lib.birkhoff_bwd(P, G, out=dfull[:B])
    torch.cuda.synchronize()
    assert torch.all(Pfull[B:] == SENTINEL) and torch.all(dfull[B:] == SENTINEL)
    rng = np.random.Generator(np.random.PCG64(2702))
    boundary = (1 << 27)  # 16 * 2^27 = 2^31: the first matrix past int32 offsets
    idx = np.unique(np.concatenate([rng.choice(B, 2048, replace=False), np.arange(B - 64, B),
                                    np.arange(boundary - 32, boundary + 32), np.arange(0, 16)]))
    ti = torch.from_numpy(idx).cuda()
    A_s = A[ti].cpu().numpy().astype(np.float64)
    P_s = P[ti].cpu().numpy().astype(np.float64)
    G_s = G[ti].cpu().numpy().astype(np.float64)
    d_s = dfull[ti].cpu().numpy().astype(np.float64)
    ok = it[ti].cpu().numpy() != 255
    ref = birkhoff_project(A_s)
    err = np.abs(P_s - ref).max(axis=(1, 2))
    assert err[ok].max() <= 1e-5, f"P error {err[ok].max():.2e}"
    dref = birkhoff_project_bwd(ref, G_s)
    tol = 1e-4 * np.abs(dref).max(axis=(1, 2)) + 1e-5 * np.abs(G_s).max(axis=(1, 2))
    ratio = np.abs(d_s - dref).max(axis=(1, 2)) / tol
    assert ratio[ok].max() <= 1.0, f"gradient error {ratio[ok].max():.3f} x tolerance"
    del A, Pfull, P, G, dfull
    torch.cuda.empty_cache()


def test_stream_mix_past_int32_offsets(gpu_lib):
    T, C = 70_000, 8192           # T * 4 * C > 2^31 elements
    print(f"large stream mix T={T} C={C}", flush=True)
    x, logits = W.mix_inputs(T, C, seed=2703)
    yfull = torch.full((T + 4, 4, C), SENTINEL, dtype=torch.bfloat16, device="cuda")
    H = torch.empty_like(logits)
    gpu_lib.ops.stream_mix_into(x, logits, H, yfull[:T])
    torch.cuda.synchronize()
    sentinel = torch.tensor(SENTINEL, dtype=torch.bfloat16, device="cuda")
    assert torch.all(yfull[T:] == sentinel)
    rng = np.random.Generator(np.random.PCG64(2704))
    per_token = 4 * C
    boundary = (1 << 31) // per_token  # token holding the 2^31-th element
    idx = np.unique(np.concatenate([rng.choice(T, 48, replace=False), np.arange(T - 4, T),
                                    np.arange(boundary - 2, boundary + 3)]))
    ti = torch.from_numpy(idx).cuda()
    Hs = H[ti].cpu().numpy().astype(np.float64)
    Href = birkhoff_project(logits[ti].cpu().numpy().astype(np.float64))
    assert np.abs(Hs - Href).max() <= 1e-5
    xs = x[ti].float().cpu().numpy().astype(np.float64)
    ys = yfull[ti].float().cpu().numpy().astype(np.float64)
    ref = stream_mix(Hs, xs)
    mag = np.einsum("tij,tjc->tic", np.abs(Hs), np.abs(xs))
    err = np.abs(ys - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * mag).all()
    del x, logits, yfull, H
    torch.cuda.empty_cache()
