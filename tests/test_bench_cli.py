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
