#!/usr/bin/env python3
"""Benchmark of the mHC Birkhoff-projection hot path on one MI355X.

Default (the headline): forward + backward projection of 131072 4x4 fp32
logit matrices drawn N(0,10^2) (seed 2), with upstream gradients N(0,1).  One
"step" is one forward launch plus one backward launch over the whole batch.
Inputs and outputs rotate over enough buffer sets (> 512 MiB) that every step
reads from HBM rather than from the 256 MB last-level cache.

Prints one JSON line:
  value        projections per second (fwd+bwd), whole job
  roofline     for the dominant kernel, the forward solve: its algorithmic
               bytes per launch (128 per matrix) / its average HIP-event
               duration, against 8 TB/s, with the counter-measured HBM bytes
               as `traffic`.  The kernel reaches neither that roof nor the
               vector-ALU one (`roofline.valu` gives its issue-slot fraction):
               it is limited by latency -- one generation of waves, two per
               SIMD, whose load phase no solve overlaps
  hbm          algorithmic GB/s of fwd, bwd and the step against 8 TB/s, and
               the counter-measured HBM bytes per launch
  iters        Newton iterations per matrix and per wave (divergence)
  overlapped   the same steps with batch k's forward and batch k-1's
               backward in one launch (mhc_birkhoff_pipeline_step; beside
               the headline, never as it)
  config3      the same fwd+bwd step on 1,048,576 mixed-difficulty matrices,
               timed in the same run (the other end of the 128K-1M range)
  cpu_baseline the float64 oracle (fwd+bwd) on the host cores, on a bounded
               sample of the same batch

Other workloads (--config 1/3/4/5) print the same kind of line for that
workload; they are not the headline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Vector ALU issue peak of MI355X: the published fp32 vector rate, 157.3
# TFLOP/s, is 157.3e12 / (64 lanes x 2 flops) = 1.229e12 wave64 FMA
# instructions per second; every VALU instruction takes one such issue slot
# and a transcendental (exp2, log2, rcp) four (quarter rate, measured).
VALU_PEAK_SLOTS = 157.3e12 / 128.0
TRANS_SLOTS = 4
FWD_BYTES = 128   # per matrix: 64 B logits in, 64 B P out
BWD_BYTES = 192   # per matrix: P and dL/dP in, dL/dA out
# Dense bf16 MFMA peak of MI355X (no sparsity), and the flops of one
# v_mfma_f32_16x16x32_bf16 instruction (2 x 16 x 16 x 32).
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FLOPS_PER_INSTR = 2 * 16 * 16 * 32
# Host cores a one-GPU machine gives this process: the CPU baselines run at most
# this many worker processes, whatever the machine's own count.
CPU_SHARE = 16
# Cycles of the bounded spin kernel queued ahead of each timed region (see
# spin_ahead).
SPIN_CYCLES = 1_000_000


def spin_ahead(torch):
    """Queue a short spin kernel (about 0.5 ms) before a timed region's start
    event, so that the GPU is busy while the host submits the region's work
    instead of idling between the start event and the first kernel.  At 20
    steps of the 131072-matrix step this measured 14.0 us per step against
    14.45 without it; 200 steps read 13.7 either way (a region still carries
    a few microseconds of fixed cost at its end).  Much longer spins read
    slower.  The spin ends after a fixed cycle count; it waits on nothing."""
    torch.cuda._sleep(SPIN_CYCLES)

# Per-launch figures from rocprofv3 counter runs (profiles/ holds the
# summaries and the commands): HBM bytes from FETCH_SIZE and WRITE_SIZE, each
# scaled by what the counter reads for a plain copy of known size, and VALU
# instructions (SQ_INSTS_VALU, of which SQ_INSTS_VALU_TRANS_F32 are
# transcendental).  They hold only for the kernel sources they were taken on:
# each entry carries the hash of the code (comments stripped) of the csrc
# files its kernels are built from (KERNEL_SOURCES), and a mismatch reports it
# as null.
KERNEL_SOURCES = {
    "proj": ("devmath.h", "proj4.h", "stage.h", "birkhoff.hip"),
    "projn": ("devmath.h", "proj4.h", "projn.h", "stage.h", "birkhoffn.hip"),
    "mix": ("devmath.h", "proj4.h", "wave.h", "mix.hip"),
    "layer": ("devmath.h", "proj4.h", "wave.h", "kernels.h", "layer.hip"),
}
MEASURED = {
    "birkhoff_fwd_131072_cfg2": {"fetch": 8530011, "write": 8388960, "valu": 2077837, "trans": 122619, "sha": "02f6a806bc3f5d91"},
    "birkhoff_bwd_131072_cfg2": {"fetch": 16805842, "write": 8388702, "valu": 1122304, "trans": 24576, "sha": "02f6a806bc3f5d91"},
    "birkhoff_pipeline_131072_cfg2": {"fetch": 25360205, "write": 16777267, "valu": 2649196, "trans": 128763, "sha": "02f6a806bc3f5d91"},
    "birkhoff_fwd_1048576_cfg3": {"fetch": 67250930, "write": 67118441, "valu": 16073142, "trans": 945927, "sha": "02f6a806bc3f5d91"},
    "birkhoff_bwd_1048576_cfg3": {"fetch": 134231236, "write": 67109184, "valu": 8978432, "trans": 196608, "sha": "02f6a806bc3f5d91"},
    "birkhoff_pipeline_1048576_cfg3": {"fetch": 201504454, "write": 134222219, "valu": 20644003, "trans": 995079, "sha": "02f6a806bc3f5d91"},
    "birkhoff_fwd_bwd_131072_cfg2": {"fetch": 16973961, "write": 16777430, "valu": 2583660, "trans": 128763, "sha": "02f6a806bc3f5d91"},
    "birkhoff_fwd_n8_131072_cfg2": {"fetch": 33951814, "write": 35652001, "valu": 20632142, "trans": 696051, "sha": "90455b546a1d0f2d"},
    "birkhoff_bwd_n8_131072_cfg2": {"fetch": 67447617, "write": 33555119, "valu": 6424576, "trans": 14336, "sha": "90455b546a1d0f2d"},
    "stream_mix_fwd_16384x4x4096": {"fetch": 539059096, "write": 537927787, "valu": 25592832, "trans": 68608, "sha": "f5dd6de6be0f8ebe"},
    "stream_mix_bwd_16384x4x4096": {"fetch": 1074714477, "write": 537950805, "valu": 49479680, "trans": 0, "sha": "f5dd6de6be0f8ebe"},
    "layer_step_65536x4x7168": {"fetch": 30741360653, "write": 9469181389, "mfma": {"layer_maps_kernel<0>": 7340032, "layer_dx_kernel": 14680064, "layer_dw_kernel": 14680064}, "us": {"layer_maps_kernel<0>": 670.64, "layer_dx_kernel": 2583.42, "layer_dw_kernel": 754.73}, "sha": "a54d06b4171c20b2"},
}


def source_group(key):
    if key.startswith(("birkhoff_fwd_n", "birkhoff_bwd_n")):
        return "projn"
    if key.startswith("birkhoff_"):
        return "proj"
    return "mix" if key.startswith("stream_mix") else "layer"


def code_text(src):
    """Source text with comments and layout removed: what the compiler sees.
    (The kernel sources hold no string literal with a comment marker.)"""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    lines = (" ".join(l.split()) for l in src.splitlines())
    return "\n".join(l for l in lines if l)


def sources_sha(group):
    """Hash of the code (not the comments) of the kernel sources of `group`."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "birkhoff_projection_amd", "csrc")
    for f in KERNEL_SOURCES[group]:
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured(key):
    """Counter-derived per-launch figures for `key`, or None if its kernel
    sources changed since they were taken."""
    m = MEASURED.get(key)
    if m is None or m.get("sha") != sources_sha(source_group(key)):
        return None
    return m


def _cpu_worker(args):
    import oracle
    A, G = args
    P = oracle.birkhoff_project(A.astype(np.float64))
    oracle.birkhoff_project_bwd(P, G.astype(np.float64))
    return A.shape[0]


def host_cores():
    """(worker processes used, cores visible to this process)."""
    visible = len(os.sched_getaffinity(0))
    return min(visible, CPU_SHARE), visible


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: report unknown
        return None


def cpu_baseline_projection(A, G, n_sample, label):
    """Time the oracle's fwd+bwd on n_sample matrices (the batch repeated if
    n_sample exceeds it) over a process pool on the host cores."""
    import multiprocessing as mp
    cores, visible = host_cores()
    n = n_sample
    idx = np.arange(n) % A.shape[0]
    chunks = np.array_split(idx, cores * 4)
    work = [(A[c], G[c]) for c in chunks]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = sum(pool.map(_cpu_worker, work))
    dt = time.perf_counter() - t0
    # one process alone, on the first 16384 matrices
    n1 = min(16384, A.shape[0])
    t1 = time.perf_counter()
    _cpu_worker((A[:n1], G[:n1]))
    dt1 = time.perf_counter() - t1
    return {"value": done / dt, "unit": "projections/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} matrices ({done / A.shape[0]:g} passes over the {A.shape[0]} "
                      f"{label} batch), fwd+bwd, float64, {dt:.1f} s wall on {cores} processes",
            "single_core": {"value": n1 / dt1, "sample": f"first {n1} matrices, one process"},
            "host_cores_visible": visible,
            "pool_note": f"process pool capped at the {CPU_SHARE}-core host share of one GPU",
            "blas_threads": _blas_threads()}


# Host copy of the token sample the per-token CPU baselines run on; worker
# processes inherit it through fork and receive only index ranges.
_TOKENS = None


def _cpu_tokens_worker(args):
    """Oracle on one range of the token sample, one BLAS thread per process:
    'mix' = projection + stream mix (the fused workload), 'layer' = layer
    step forward + backward."""
    import oracle
    from threadpoolctl import threadpool_limits
    kind, lo, hi = args
    with threadpool_limits(1):
        if kind == "mix":
            x, logits = _TOKENS
            H = oracle.birkhoff_project(logits[lo:hi].astype(np.float64))
            oracle.stream_mix(H, x[lo:hi].astype(np.float64))
        else:
            x, Wm, f, dxo, du = _TOKENS
            x64, W64, f64 = (a.astype(np.float64) for a in (x[lo:hi], Wm, f[lo:hi]))
            fw = oracle.layer_fwd(x64, W64, f64)
            oracle.layer_bwd(x64, W64, f64, dxo[lo:hi].astype(np.float64),
                             du[lo:hi].astype(np.float64), fwd=fw)
    return hi - lo


def cpu_baseline_tokens(kind, tokens, n, T_total, label):
    """Per-token oracle throughput on the first ``n`` tokens of the host
    sample ``tokens`` (a tuple of float32 arrays, the workload's own inputs)
    over a process pool; the tokens/s is the sample's, and the whole
    workload's time is extrapolated from it and labelled as such."""
    import multiprocessing as mp
    global _TOKENS
    cores, visible = host_cores()
    _TOKENS = tokens
    bounds = np.linspace(0, n, 4 * cores + 1).astype(int)
    work = [(kind, int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        t0 = time.perf_counter()
        done = sum(pool.map(_cpu_tokens_worker, work))
        dt = time.perf_counter() - t0
    _TOKENS = None
    rate = done / dt
    return {"value": rate, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {done} of the {T_total} tokens ({label}), float64, "
                      f"{dt:.1f} s wall on {cores} processes with one BLAS thread each"
                      + (f"; extrapolated, the whole workload would take {T_total / rate:.0f} s"
                         if done < T_total else ""),
            "extrapolated": done < T_total, "host_cores_visible": visible,
            "pool_note": f"process pool capped at the {CPU_SHARE}-core host share of one GPU"}


def time_projection(bp, torch, A_np, G_np, steps, warmup, solver="newton", recompute=False, n=4,
                    fused=False, overlap=False):
    """Rotate over buffer sets and time `steps` fwd+bwd steps back to back,
    then `steps` forward launches alone and `steps` backward launches alone.

    Each timed sequence is captured once into a HIP graph and replayed: at
    this size a kernel takes 7-15 us, about what one call through the Python
    binding costs on the host, so eager launches would time the host.  Before
    timing, the step graph is replayed twice with eager work in between and
    every buffer set's P and dA are compared bit for bit with the same
    projections run eagerly.  The eager rate is reported too.  HIP events on
    the replay stream bracket each replay, so a kernel's average is its
    duration plus the inter-kernel gap, comparable with a kernel trace."""
    B = A_np.shape[0]
    set_bytes = B * n * n * 4 * 4
    nsets = max(2, int(np.ceil(600e6 / set_bytes)))
    fwd_fn = bp.birkhoff_fwd if n == 4 else bp.birkhoff_fwd_n
    bwd_fn = bp.birkhoff_bwd if n == 4 else bp.birkhoff_bwd_n
    A0 = torch.from_numpy(A_np).cuda()
    G0 = torch.from_numpy(G_np).cuda()
    sets = []
    for _ in range(nsets):
        sets.append((A0.clone(), torch.empty_like(A0), G0.clone(), torch.empty_like(A0)))

    def fwd(k):
        A, P, G, dA = sets[k % nsets]
        if fused:  # P and dA in one launch
            bp.birkhoff_fwd_bwd(A, G, out_P=P, out_grad=dA, solver=solver)
        else:
            fwd_fn(A, out=P, solver=solver)

    def bwd(k):
        A, P, G, dA = sets[k % nsets]
        if fused:
            return
        if recompute:
            bp.birkhoff_bwd_recompute(A, G, out=dA, solver=solver)
        else:
            bwd_fn(P, G, out=dA)

    def step(k):
        fwd(k)
        bwd(k)

    # Pipelined schedule: one launch runs the forward of batch k and the
    # backward of batch k-1 (mhc_birkhoff_pipeline_step), as a trainer that
    # overlaps micro-batches would; a forward alone opens the sequence and a
    # pipeline launch with an empty forward closes it.  Every batch still
    # gets its forward, then its backward, and stream order alone keeps the
    # dependencies: launch k writes P of set k and reads P of set k-1
    # (nsets >= 2).
    no_fwd = torch.empty((0, 4, 4), dtype=torch.float32, device=A0.device)

    def pipelined():
        fwd(0)
        for k in range(1, steps):
            A, P, G, dA = sets[k % nsets]
            Ap, Pp, Gp, dAp = sets[(k - 1) % nsets]
            bp.birkhoff_pipeline_step(A, Pp, Gp, out=P, out_grad=dAp, solver=solver)
        # the last backward from the same kernel, its forward half empty
        A, P, G, dA = sets[(steps - 1) % nsets]
        bp.birkhoff_pipeline_step(no_fwd, P, G, out=no_fwd, out_grad=dA, solver=solver)

    def events():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def eager(body):
        start, stop = events()
        torch.cuda.synchronize()
        spin_ahead(torch)
        start.record()
        for k in range(steps):
            body(k)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop)

    def capture(body, whole=False):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if whole:
                body()
            else:
                for k in range(steps):
                    body(k)
        torch.cuda.synchronize()
        return g

    def replay(g):
        start, stop = events()
        torch.cuda.synchronize()
        spin_ahead(torch)
        start.record()
        g.replay()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop)

    for k in range(warmup):
        step(k)
    eager_ms = eager(step)
    g_step, g_fwd = capture(step), capture(fwd)
    g_bwd = None if fused else capture(bwd)  # fused: nothing left to time apart
    # replays must reproduce the eager results exactly (deterministic kernels);
    # the captured steps write the first min(steps, nsets) buffer sets
    touched = sets[:min(steps, nsets)]
    ref = []
    for A, P, G, dA in touched:
        if fused:
            Pe, dAe = bp.birkhoff_fwd_bwd(A, G, solver=solver)
        else:
            Pe = fwd_fn(A, solver=solver)
            dAe = bp.birkhoff_bwd_recompute(A, G, solver=solver) if recompute else bwd_fn(Pe, G)
        ref.append((Pe, dAe))
    g_over = capture(pipelined, whole=True) if overlap else None
    # the pipeline launch forms the gradient one matrix per lane, bit for bit
    # the recompute backward's for the same logits
    ref_over = ([(Pe, bp.birkhoff_bwd_recompute(A, G, solver=solver))
                 for (A, P, G, dA), (Pe, dAe) in zip(touched, ref)] if overlap else None)
    for g, refs in ((g_step, ref), (g_over, ref_over)):
        if g is None:
            continue
        for _ in range(2):
            for A, P, G, dA in touched:
                P.zero_()
                dA.zero_()
            g.replay()
            torch.cuda.synchronize()
            for (A, P, G, dA), (Pe, dAe) in zip(touched, refs):
                if not (torch.equal(P, Pe) and torch.equal(dA, dAe)):
                    raise RuntimeError("graph replay differs from eager results")
            fwd_fn(sets[0][0], solver=solver)  # eager work between replays
    for _ in range(2):  # warm replays (a graph's first replays run slower)
        g_step.replay()
        g_fwd.replay()
        if g_bwd is not None:
            g_bwd.replay()
    torch.cuda.synchronize()
    total_ms = replay(g_step)  # the timed region: exactly `steps` steps
    fwd_ms = replay(g_fwd) / steps
    bwd_ms = 0.0 if fused else replay(g_bwd) / steps
    # spread: five more replays of the step graph (not part of the headline)
    spread = sorted(replay(g_step) / steps for _ in range(5))
    # hot cache: every step on the same buffer set (reported apart, never the
    # headline: the set fits in the 256 MB last-level cache)
    g_hot = capture(lambda k: step(0))
    g_hot.replay()
    g_hot.replay()
    hot_ms = replay(g_hot) / steps
    over_ms = None
    if g_over is not None:
        g_over.replay()
        g_over.replay()
        over_ms = sorted(replay(g_over) / steps for _ in range(3))[1]
    return dict(total_ms=total_ms, fwd_ms=fwd_ms, bwd_ms=bwd_ms, nsets=nsets,
                eager_ms_per_step=eager_ms / steps, step_ms_median=spread[2],
                step_ms_min=spread[0], hot_ms_per_step=hot_ms, overlapped_ms_per_step=over_ms)


def copy_bandwidth(torch, mib=256, reps=20):
    """Read+write GB/s of a plain device copy of `mib` MiB, the practical
    streaming ceiling the kernels' algorithmic GB/s is compared with."""
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        y.copy_(x)
    stop.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (start.elapsed_time(stop) / 1e3) / 1e9
    del x, y
    return gbs


def copy_probe(torch, mib):
    """One plain device copy of a known size (for scaling HBM byte counters)."""
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def iteration_stats(bp, torch, A_np, n=4):
    """Newton iterations per matrix (the kernel's own count) and the mean over
    waves of the largest count among a wave's 64 consecutive matrices: a wave
    runs until its slowest lane is done, so their ratio is the share of
    issued lane-work that is useful."""
    A = torch.from_numpy(A_np).cuda()
    _, it = (bp.birkhoff_fwd if n == 4 else bp.birkhoff_fwd_n)(A, return_iters=True)
    it = it.cpu().numpy().astype(np.int64)
    ok = it != 255
    itc = np.where(ok, it, 30)
    n = (len(itc) // 64) * 64
    wave_max = itc[:n].reshape(-1, 64).max(axis=1)
    return {"mean": float(itc.mean()), "wave_max_mean": float(wave_max.mean()),
            "useful_frac": float(itc[:n].mean() / wave_max.mean()) if wave_max.mean() > 0 else 1.0,
            "not_converged": int((~ok).sum()),
            "hist_matrix": np.bincount(it[ok], minlength=1).tolist(),
            "hist_wave_max": np.bincount(wave_max, minlength=1).tolist()}


def bench_projection(args, bp, torch, config):
    import workloads as W
    n = args.n
    if n != 4:
        if config not in (1, 2):
            raise SystemExit("--n applies to configs 1 and 2 (their shapes and distributions, n x n)")
        B = 4096 if config == 1 else 131072
        kind = "normal1" if config == 1 else "normal10"
        A = W.logits_batch(kind, B, 0 if config == 1 else 2, n=n)
        G = W.grad_batch(B, 1 if config == 1 else 3, n=n)
        label = ("N(0,1)" if config == 1 else "N(0,10^2)") + f" {n}x{n}"
    elif config == 2:
        A, G = W.config2()
        label = "N(0,10^2)"
    elif config == 3:
        A, G, _ = W.config3()
        label = "mixed-difficulty"
    else:
        A = W.config1()
        G = W.grad_batch(A.shape[0], 1)
        label = "N(0,1)"
    B = A.shape[0]
    if (args.recompute or args.fused) and n != 4:
        raise SystemExit("--recompute and --fused are for 4x4 matrices")
    if args.recompute and args.fused:
        raise SystemExit("--recompute and --fused exclude each other")
    r = time_projection(bp, torch, A, G, args.steps, args.warmup, recompute=args.recompute, n=n,
                        fused=args.fused, overlap=n == 4 and not (args.fused or args.recompute))
    ms = r["total_ms"] / args.steps
    fwd_avg = float(r["fwd_ms"])
    bwd_avg = float(r["bwd_ms"])
    value = B / (ms / 1e3)
    fwd_bytes = FWD_BYTES * n * n // 16
    bwd_bytes = BWD_BYTES * n * n // 16  # recompute: logits and dL/dP in, dL/dA out -- the same
    if args.fused:  # one kernel: logits and dL/dP in, P and dL/dA out
        fwd_bytes, bwd_bytes = 2 * FWD_BYTES, 0
    fwd_gbs = fwd_bytes * B / (fwd_avg / 1e3) / 1e9
    bwd_gbs = bwd_bytes * B / (bwd_avg / 1e3) / 1e9 if bwd_avg > 0 else None
    step_gbs = (fwd_bytes + bwd_bytes) * B / (ms / 1e3) / 1e9
    copy_gbs = copy_bandwidth(torch)
    tag = "" if n == 4 else f"_n{n}"
    fwd_key = f"birkhoff_fwd_bwd_{B}_cfg{config}" if args.fused else f"birkhoff_fwd{tag}_{B}_cfg{config}"
    kname = "birkhoff_fwd_bwd (fused Newton + backward)" if args.fused else "birkhoff_fwd (Newton)"
    m_fwd = measured(fwd_key)
    m_bwd = None if (args.recompute or args.fused) else measured(f"birkhoff_bwd{tag}_{B}_cfg{config}")
    roofline, valu = forward_roofline(kname, fwd_bytes * B, fwd_avg, B, m_fwd)
    out = {
        "metric": "4x4 projections/sec fwd+bwd at 128K batch; achieved HBM GB/s vs peak",
        "value": value, "unit": "projections/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"birkhoff fwd+bwd, {B} {n}x{n} fp32 matrices {label}",
                   "batch": B, "n": n, "solver": "newton", "tol": 1e-6,
                   "backward": ("recompute" if args.recompute else
                                "fused with the forward (dL/dP given)" if args.fused else "from P"),
                   "buffer_sets": r["nsets"]},
        "roofline": roofline,
        "hbm": {"fwd_GBs": fwd_gbs, "bwd_GBs": bwd_gbs, "step_GBs": step_gbs,
                "step_frac": step_gbs / HBM_PEAK_GBS,
                "bwd_frac": bwd_gbs / HBM_PEAK_GBS if bwd_gbs is not None else None,
                "copy_GBs": copy_gbs, "step_frac_of_copy": step_gbs / copy_gbs,
                "fwd_traffic": m_fwd["fetch"] + m_fwd["write"] if m_fwd else None,
                "bwd_traffic": m_bwd["fetch"] + m_bwd["write"] if m_bwd else None},
        "kernels": {"fwd_us": fwd_avg * 1e3, "bwd_us": bwd_avg * 1e3, "launch": "hip graph replay",
                    "eager_us_per_step": r["eager_ms_per_step"] * 1e3,
                    "step_us_median_of_5": r["step_ms_median"] * 1e3,
                    "step_us_min_of_5": r["step_ms_min"] * 1e3,
                    "hot_us_per_step": r["hot_ms_per_step"] * 1e3},
        "valu": valu,
        "iters": iteration_stats(bp, torch, A, n),
    }
    if r["overlapped_ms_per_step"] is not None:
        out["overlapped"] = overlapped_block(r, B, fwd_bytes + bwd_bytes,
                                             f"birkhoff_pipeline_{B}_cfg{config}")
    if config == 2 and n == 4 and not (args.recompute or args.fused) and not args.no_config3:
        out["config3"] = config3_block(args, bp, torch)
    if not args.no_cpu_baseline:
        sample = args.cpu_sample if n == 4 else max(args.cpu_sample * 16 // (n * n * 4), 16384)
        out["cpu_baseline"] = cpu_baseline_projection(A, G, sample, label)
    return out


def overlapped_block(r, B, step_bytes, key=None):
    """The same steps with batch k's forward and batch k-1's backward in one
    launch (mhc_birkhoff_pipeline_step; see time_projection).  Reported
    beside the headline, never as it: the headline step keeps each batch's
    forward and backward in two launches, one after the other."""
    ms = r["overlapped_ms_per_step"]
    gbs = step_bytes * B / (ms / 1e3) / 1e9
    return {"schedule": "mhc_birkhoff_pipeline_step: forward of batch k and backward of batch "
                        "k-1 in one launch (a forward alone opens the sequence, a pipeline "
                        "launch with an empty forward closes it); P bit-identical to the serial "
                        "steps', the gradient to mhc_birkhoff_bwd_recompute's (one matrix per "
                        "lane)",
            "value": B / (ms / 1e3), "unit": "projections/s", "ms_per_step": ms,
            "step_GBs": gbs, "step_frac": gbs / HBM_PEAK_GBS, "timing": "median of 3 replays",
            "traffic": (lambda m: m["fetch"] + m["write"] if m else None)(measured(key) if key else None),
            "algorithmic_bytes": step_bytes * B}


def forward_roofline(kname, alg_bytes, fwd_ms, B, m):
    """Roofline of the forward solve: algorithmic bytes per launch over its
    average duration against the HBM peak, and beside it the vector-ALU view
    (issue slots per launch from the counter run of this kernel on this
    workload, over the same duration, against the fp32 vector issue peak).
    It reaches neither roof: with one generation of waves, two per SIMD, the
    load phase of every wave finishes before any solve starts and each wave
    then runs until its slowest matrix is done (latency, not throughput)."""
    achieved = alg_bytes / (fwd_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": m["fetch"] + m["write"] if m else None,
            "algorithmic_bytes": alg_bytes, "limiter": "latency"}
    if m is None:
        roof["valu"] = None
        roof["note"] = "kernel changed since its counters were taken: traffic and VALU unknown"
        return roof, None
    slots = m["valu"] + (TRANS_SLOTS - 1) * m["trans"]
    rate = slots / (fwd_ms / 1e3)
    roof["valu"] = {"achieved": rate, "peak": VALU_PEAK_SLOTS, "unit": "wave64 VALU issue slots/s",
                    "frac": rate / VALU_PEAK_SLOTS}
    valu = {"instructions_per_launch": m["valu"], "transcendental": m["trans"],
            "issue_slots_per_launch": slots, "slots_per_matrix": slots / B}
    return roof, valu


def config3_block(args, bp, torch):
    """The fwd+bwd step on the 1,048,576-matrix mixed-difficulty batch,
    timed in the same run as the headline (same method: rotated buffer sets
    past the last-level cache, HIP-graph replay, HIP events)."""
    import workloads as W
    A, G, _ = W.config3()
    B = A.shape[0]
    r = time_projection(bp, torch, A, G, args.steps, args.warmup, overlap=True)
    ms = r["total_ms"] / args.steps
    fwd_ms, bwd_ms = float(r["fwd_ms"]), float(r["bwd_ms"])
    step_gbs = (FWD_BYTES + BWD_BYTES) * B / (ms / 1e3) / 1e9
    m_fwd = measured(f"birkhoff_fwd_{B}_cfg3")
    roof, valu = forward_roofline("birkhoff_fwd (Newton)", FWD_BYTES * B, fwd_ms, B, m_fwd)
    return {"workload": f"birkhoff fwd+bwd, {B} 4x4 fp32 matrices, mixed difficulty (50 % N(0,1), "
                        f"40 % N(0,10^2), 10 % N(0,1) + 20 I)",
            "value": B / (ms / 1e3), "unit": "projections/s", "ms_per_step": ms,
            "fwd_us": fwd_ms * 1e3, "bwd_us": bwd_ms * 1e3,
            "step_GBs": step_gbs, "step_frac": step_gbs / HBM_PEAK_GBS,
            "fwd_GBs": FWD_BYTES * B / (fwd_ms / 1e3) / 1e9,
            "bwd_GBs": BWD_BYTES * B / (bwd_ms / 1e3) / 1e9,
            "bwd_frac": BWD_BYTES * B / (bwd_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "step_us_median_of_5": r["step_ms_median"] * 1e3, "roofline_fwd": roof, "valu": valu,
            "iters": iteration_stats(bp, torch, A),
            "overlapped": overlapped_block(r, B, FWD_BYTES + BWD_BYTES, f"birkhoff_pipeline_{B}_cfg3")}


def _time_loop(torch, body, steps, warmup):
    stream = torch.cuda.current_stream()
    for k in range(warmup):
        body(k)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    spin_ahead(torch)
    start.record(stream)
    for k in range(steps):
        body(k)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def _host_tokens(idx, *tensors):
    """Host float32 copies of the given tokens of each device tensor."""
    return tuple(t[idx].float().cpu().numpy() for t in tensors)


def bench_mix(args, bp, torch):
    """Fused projection + stream mix, T=16384, C=4096 (logits N(0,2^2))."""
    import workloads as W
    T, C = W.CONFIG4_SHAPE["T"], W.CONFIG4_SHAPE["C"]
    x, logits = W.mix_inputs(T, C, seed=4)
    y = torch.empty_like(x)
    H = torch.empty_like(logits)
    ms = _time_loop(torch, lambda k: bp.ops.stream_mix_into(x, logits, H, y), args.steps, args.warmup)
    per_tok = 64 + 4 * C * 2 + 64 + 4 * C * 2
    gbs = per_tok * T / (ms / 1e3) / 1e9
    m = measured(f"stream_mix_fwd_{T}x4x{C}")
    traffic = m["fetch"] + m["write"] if m else None
    out = {
        "metric": "fused projection + stream mix tokens/s; achieved HBM GB/s vs peak",
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"fused projection + stream mix, T={T}, n=4, C={C} bf16"},
        "roofline": {"bound": "hbm", "kernel": "stream_mix_fwd (fused Newton)", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": per_tok * T,
                     "traffic_ratio": traffic / (per_tok * T) if traffic else None},
    }
    if not args.no_cpu_baseline:
        n = min(T, args.cpu_tokens_mix)
        out["cpu_baseline"] = cpu_baseline_tokens("mix", _host_tokens(slice(0, n), x, logits), n, T,
                                                  "projection of the logits + stream mix")
    return out


def bench_mix_bwd(args, bp, torch):
    """Stream-mix backward alone (mhc_stream_mix_bwd), T=16384, C=4096: the
    standalone call; the layer step uses its own backward passes."""
    import workloads as W
    T, C = W.CONFIG4_SHAPE["T"], W.CONFIG4_SHAPE["C"]
    x, dout, logits = W.mix_bwd_inputs(T, C, seed=44)
    H = bp.birkhoff_fwd(logits)
    gx, gH = torch.empty_like(x), torch.empty_like(H)
    ms = _time_loop(torch, lambda k: bp.stream_mix_bwd(x, H, dout, out=(gx, gH)), args.steps,
                    args.warmup)
    per_tok = 3 * (4 * C * 2) + 64 + 64  # x, grad_out in, grad_x out; H in, grad_H out
    gbs = per_tok * T / (ms / 1e3) / 1e9
    m = measured(f"stream_mix_bwd_{T}x4x{C}")
    return {
        "metric": "stream mix backward tokens/s; achieved HBM GB/s vs peak",
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"stream mix backward, T={T}, n=4, C={C} bf16"},
        "roofline": {"bound": "hbm", "kernel": "stream_mix_bwd", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": m["fetch"] + m["write"] if m else None},
    }


# Layer-step kernels with MFMA work: (key in MEASURED, v_mfma_f32_16x16x32_bf16
# instructions per launch counted by SQ_INSTS_MFMA, traced average duration in
# us, useful GEMM flops per launch).  Useful flops at T tokens, width C: the
# map GEMM 2 T 24 (4C); dx's dl W and dw's dl^T x the same each, counted once
# although both feed dl as a bf16 hi + lo pair (two MFMAs per product).
LAYER_MFMA_KERNELS = ("layer_maps_kernel<0>", "layer_dx_kernel", "layer_dw_kernel")


def layer_mfma(T, C, m):
    """MFMA utilisation of the layer's three contraction kernels from the
    counter run (instructions) and the kernel trace (durations) stored for
    this workload; None when the kernel sources changed since."""
    if m is None or "mfma" not in m:
        return None
    useful = 2.0 * T * 24 * 4 * C
    res = {}
    for name in LAYER_MFMA_KERNELS:
        instr, us = m["mfma"][name], m["us"][name]
        issued = instr * MFMA_FLOPS_PER_INSTR / (us * 1e-6) / 1e12
        res[name] = {"mfma_instructions": instr, "traced_us": us,
                     "issued_TFLOPs": issued, "issued_frac": issued / MFMA_BF16_PEAK_TFLOPS,
                     "useful_TFLOPs": useful / (us * 1e-6) / 1e12,
                     "useful_frac": useful / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    res["peak_TFLOPs"] = MFMA_BF16_PEAK_TFLOPS
    res["note"] = ("v_mfma_f32_16x16x32_bf16 count x 16384 flops over the traced duration "
                   "(profiles/layer_step_65536x4x7168.md); HBM-bound kernels, reported, not chased")
    return res


def bench_layer(args, bp, torch):
    """Full layer step fwd+bwd, T=65536, n=4, C=7168."""
    import workloads as W
    T, C = W.CONFIG5_SHAPE["T"], W.CONFIG5_SHAPE["C"]
    inp = W.layer_inputs(T, C, seed=5)
    x, Wt, f, dxo, du = inp["x"], inp["W"], inp["f"], inp["dx_out"], inp["du"]
    fw = bp.layer_fwd(x, Wt, f)
    ws = bp.layer_workspace(T, C, x.device)
    bw = bp.layer_bwd(x, Wt, f, fw, dxo, du, workspace=ws)
    torch.cuda.synchronize()
    fwd_ms = _time_loop(torch, lambda k: bp.ops.layer_fwd_into(x, Wt, f, fw), args.steps, args.warmup)
    bwd_ms = _time_loop(torch, lambda k: bp.layer_bwd(x, Wt, f, fw, dxo, du, workspace=ws, out=bw),
                        args.steps, args.warmup)
    ms = fwd_ms + bwd_ms
    D = 4 * C
    # Algorithmic bytes of the step: forward reads x twice (the maps need the
    # whole token row before any map is known) and f, writes u and x_out,
    # plus the 196 bytes of per-token maps; backward reads x, grad_x_out, f
    # and grad_u once and writes grad_x and grad_f once.
    fwd_alg = T * (2 * (2 * D) + 2 * C + 2 * C + 2 * D + 196)
    bwd_alg = T * (2 * D + 2 * D + 2 * C + 2 * C + 2 * D + 2 * C)
    alg = fwd_alg + bwd_alg
    gbs = alg / (ms / 1e3) / 1e9
    # bytes this implementation's passes move (it reads x three times and
    # grad_x_out, grad_u twice in the backward)
    pass_bytes = (T * (2 * D + 196 + 2 * D + 2 * C + 2 * C + 2 * D)
                  + T * (2 * D + 2 * D + 2 * C + 2 * C + 2 * D + 2 * D + 2 * C + 2 * D + 2 * C + 2 * D))
    m = measured(f"layer_step_{T}x4x{C}")
    traffic = m["fetch"] + m["write"] if m else None
    out = {
        "metric": "mHC layer step fwd+bwd tokens/s; achieved HBM GB/s vs peak",
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"mHC layer step fwd+bwd, T={T}, n=4, C={C} bf16, W [24, {D}]"},
        "roofline": {"bound": "hbm", "kernel": "whole step (2 forward + 5 backward kernels)",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg,
                     "traffic_ratio": traffic / alg if traffic else None},
        "kernels": {"fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                    "fwd_GBs": fwd_alg / (fwd_ms / 1e3) / 1e9,
                    "bwd_GBs": bwd_alg / (bwd_ms / 1e3) / 1e9,
                    "fwd_frac": fwd_alg / (fwd_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "bwd_frac": bwd_alg / (bwd_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "pass_bytes": pass_bytes,
                    "pass_GBs": pass_bytes / (ms / 1e3) / 1e9},
        "mfma": layer_mfma(T, C, m),
    }
    if not args.no_cpu_baseline:
        n = min(T, args.cpu_tokens_layer)
        xh, fh, dxoh, duh = _host_tokens(slice(0, n), x, f, dxo, du)
        out["cpu_baseline"] = cpu_baseline_tokens(
            "layer", (xh, Wt.float().cpu().numpy(), fh, dxoh, duh), n, T,
            "layer step forward + backward")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-sample", type=int, default=2097152,
                    help="matrices the oracle baseline processes (about 10-30 s of CPU work)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain copy of this size first (counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens-mix", type=int, default=16384,
                    help="config 4: tokens of the per-token oracle baseline (16384: all of them)")
    ap.add_argument("--cpu-tokens-layer", type=int, default=16384,
                    help="config 5: tokens of the per-token oracle baseline, extrapolated to "
                         "the 65536 of the workload")
    ap.add_argument("--no-config3", action="store_true",
                    help="config 2: skip the 1M-matrix block timed beside the headline")
    ap.add_argument("--n", type=int, default=4, choices=range(1, 9), metavar="N",
                    help="configs 1-2: n x n matrices (1..8) through mhc_birkhoff_fwd_n/bwd_n")
    ap.add_argument("--mix-bwd", action="store_true",
                    help="config 4: time the standalone stream-mix backward instead")
    ap.add_argument("--fused", action="store_true",
                    help="configs 1-3, 4x4: time mhc_birkhoff_fwd_bwd, P and the gradient in one "
                         "launch for a dL/dP known at forward time (not a training step; never "
                         "the headline)")
    ap.add_argument("--recompute", action="store_true",
                    help="configs 1-3: backward by mhc_birkhoff_bwd_recompute (logits and "
                         "dL/dP in, the projection solved again; P not kept)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every batch element is independent, so the "
              "path shards by splitting the batch with no exchange; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import birkhoff_projection_amd as bp
    bp.lib()
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
    if args.config == 4:
        out = bench_mix_bwd(args, bp, torch) if args.mix_bwd else bench_mix(args, bp, torch)
    elif args.config == 5:
        out = bench_layer(args, bp, torch)
    else:
        out = bench_projection(args, bp, torch, args.config)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
