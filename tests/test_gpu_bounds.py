"""Every call writes exactly its own batch.  Outputs are views of the head of
larger buffers whose tail holds a sentinel; after the call the tail must be
unchanged and the head fully written.  The batch sizes end inside a wave
(1, 63, 65), inside a workgroup (1000) and on a wave boundary (128), which
exercises the partial-wave paths of the staged record stores."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0
EXTRA = 300  # records past the batch


def _out(B, shape_tail, dtype=torch.float32):
    full = torch.full((B + EXTRA,) + shape_tail, SENTINEL, dtype=dtype, device="cuda")
    return full, full[:B]


def _check(full, B, label):
    torch.cuda.synchronize()
    sentinel = torch.tensor(SENTINEL, dtype=full.dtype, device=full.device)  # as stored
    assert torch.all(full[B:] == sentinel), f"{label}: wrote past the batch"
    head = full[:B]
    assert torch.isfinite(head.float()).all(), f"{label}: output not fully written"
    assert not torch.any(head == sentinel), f"{label}: output not fully written"


@pytest.mark.parametrize("B", [1, 63, 65, 128, 1000])
def test_projection_4x4_writes_only_its_batch(gpu_lib, B):
    print(f"bounds 4x4 B={B}", flush=True)
    A = torch.from_numpy(W.logits_batch("normal10", B, 500 + B)).cuda()
    G = torch.from_numpy(W.grad_batch(B, 600 + B)).cuda()
    P = gpu_lib.birkhoff_fwd(A)
    calls = {
        "fwd newton": lambda out: gpu_lib.birkhoff_fwd(A, out=out),
        "fwd sinkhorn": lambda out: gpu_lib.birkhoff_fwd(A, out=out, solver="sinkhorn"),
        "bwd": lambda out: gpu_lib.birkhoff_bwd(P, G, out=out),
        "bwd recompute": lambda out: gpu_lib.birkhoff_bwd_recompute(A, G, out=out),
    }
    for label, call in calls.items():
        full, head = _out(B, (4, 4))
        call(head)
        _check(full, B, label)
    fullP, headP = _out(B, (4, 4))
    fullD, headD = _out(B, (4, 4))
    gpu_lib.birkhoff_fwd_bwd(A, G, out_P=headP, out_grad=headD)
    _check(fullP, B, "fused fwd+bwd P")
    _check(fullD, B, "fused fwd+bwd dA")
    # pipeline step: the forward and the backward batch of different sizes
    Bo = B + 37
    Ao = torch.from_numpy(W.logits_batch("normal10", Bo, 900 + B)).cuda()
    fullP, headP = _out(Bo, (4, 4))
    fullD, headD = _out(B, (4, 4))
    gpu_lib.birkhoff_pipeline_step(Ao, P, G, out=headP, out_grad=headD)
    _check(fullP, Bo, "pipeline P")
    _check(fullD, B, "pipeline dA")


@pytest.mark.parametrize("n", [2, 3, 5, 8])
@pytest.mark.parametrize("B", [1, 65, 1000])
def test_projection_n_writes_only_its_batch(gpu_lib, n, B):
    print(f"bounds n={n} B={B}", flush=True)
    A = torch.from_numpy(W.logits_batch("normal10", B, 700 + B, n=n)).cuda()
    G = torch.from_numpy(W.grad_batch(B, 800 + B, n=n)).cuda()
    P = gpu_lib.birkhoff_fwd_n(A)
    for label, call in (("fwd_n", lambda out: gpu_lib.birkhoff_fwd_n(A, out=out)),
                        ("bwd_n", lambda out: gpu_lib.birkhoff_bwd_n(P, G, out=out))):
        full, head = _out(B, (n, n))
        call(head)
        _check(full, B, f"{label} n={n}")


@pytest.mark.parametrize("T", [1, 17])
def test_stream_mix_writes_only_its_tokens(gpu_lib, T):
    print(f"bounds stream mix T={T}", flush=True)
    C = 256
    x, logits = W.mix_inputs(T, C, seed=900 + T)
    H_full, H_head = _out(T, (4, 4))
    y_full, y_head = _out(T, (4, C), dtype=torch.bfloat16)
    gpu_lib.ops.stream_mix_into(x, logits, H_head, y_head)
    _check(H_full, T, "stream mix H")
    _check(y_full, T, "stream mix out")
