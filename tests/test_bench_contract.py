"""bench.py's command-line contract, checked without a GPU: more than one GPU is refused
with a message (the measurement is one GPU's), and a machine without a GPU gets an error
rather than a CPU fallback."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=600, env=env)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = run(env=env)
    assert r.returncode == 2 and r.stdout == ""


def test_no_gpu_no_fallback():
    import torch
    if torch.cuda.is_available():
        return  # the GPU suite runs the bench itself
    r = run("--steps", "1", "--warmup", "0", "--no-decode", "--no-cpu")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_reports_the_processes_it_used():
    """The oracle baseline runs one single-threaded process per worker and reports that
    count as its cores; every worker has exited when it returns."""
    import multiprocessing as mp
    sys.path.insert(0, ROOT)
    import bench
    r = bench.cpu_baseline(64, 2, 2)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert r["host_cores"] >= 1
    assert mp.active_children() == []
