"""bench.py's command-line contract, checked without a GPU: more than one
GPU is refused with a message, --help lists the workloads, and the stored
counter figures are well formed (each names a source group whose files
exist; whether they are current is bench.py's own check at run time)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--config", "--steps", "--warmup", "--n", "--fused", "--recompute", "--mix-bwd"):
        assert flag in r.stdout


def test_stored_counters_are_well_formed():
    import bench
    for key, m in bench.MEASURED.items():
        assert {"fetch", "write", "sha"} <= set(m), key
        assert m["fetch"] > 0 and m["write"] > 0, key
        group = bench.source_group(key)
        for f in bench.KERNEL_SOURCES[group]:
            assert os.path.exists(os.path.join(ROOT, "birkhoff_projection_amd", "csrc", f)), f




def test_stored_counters_match_the_sources():
    """Every stored counter entry was taken on the kernel code as it stands
    (a code change without retaking the counters would make the bench report
    traffic and instruction counts as unknown)."""
    import bench
    stale = [k for k in bench.MEASURED if bench.measured(k) is None]
    assert not stale, f"counters taken on other kernel code: {stale}"

def test_counter_hash_ignores_comments_only():
    """The stored counters are keyed by the code of the kernel sources: a
    comment or layout change keeps the key, a code change does not."""
    import bench
    a = "int f(int x) {  // doubles\n  return 2 * x; /* why */\n}\n"
    b = "// a header note\nint f(int x) {\n\n    return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert "doubles" not in bench.code_text(a) and "why" not in bench.code_text(a)

def test_cpu_baselines_and_roofline_helpers():
    """The per-token oracle baselines of configs 4 and 5 and the projection
    baseline run on small host samples and report what they used; the
    forward roofline is algorithmic bytes over time against 8 TB/s."""
    import numpy as np
    import bench
    import workloads as W
    g = np.random.Generator(np.random.PCG64(5))
    T, C = 32, 64
    x = g.standard_normal((T, 4, C)).astype(np.float32)
    logits = (2 * g.standard_normal((T, 4, 4))).astype(np.float32)
    mix = bench.cpu_baseline_tokens("mix", (x, logits), T, 16384, "test")
    assert mix["value"] > 0 and mix["unit"] == "tokens/s" and mix["extrapolated"]  # 32 of 16384
    assert 1 <= mix["cores"] <= bench.CPU_SHARE and mix["host_cores_visible"] >= mix["cores"]
    Wm = (0.02 * g.standard_normal((24, 4 * C))).astype(np.float32)
    f, du = (g.standard_normal((T, C)).astype(np.float32) for _ in range(2))
    dxo = g.standard_normal((T, 4, C)).astype(np.float32)
    lay = bench.cpu_baseline_tokens("layer", (x, Wm, f, dxo, du), T, 65536, "test")
    assert lay["value"] > 0 and "32 of the 65536 tokens" in lay["sample"]
    A = W.logits_batch("normal10", 256, 1)
    G = W.grad_batch(256, 2)
    proj = bench.cpu_baseline_projection(A, G, 512, "test")
    assert proj["value"] > 0 and proj["unit"] == "projections/s"
    roof, valu = bench.forward_roofline("k", 128 * 131072, 0.008, 131072, None)
    assert roof["bound"] == "hbm" and abs(roof["achieved"] - 128 * 131072 / 8e-6 / 1e9) < 1e-6
    assert abs(roof["frac"] - roof["achieved"] / 8000.0) < 1e-12 and valu is None
    m = {"fetch": 1, "write": 2, "valu": 1000, "trans": 10}
    roof, valu = bench.forward_roofline("k", 1024, 0.001, 8, m)
    assert roof["traffic"] == 3 and valu["issue_slots_per_launch"] == 1030
