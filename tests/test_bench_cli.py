"""bench.py's command line on the CPU: the one-GPU scope is enforced before
any device is touched, and the help text names every workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    # The path needs no cross-GPU exchange; --gpus N > 1 exits with status 2
    # and says so, without printing a JSON line.
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for key in ("c1", "c5", "--settle-ms", "--min-rotation-mib"):
        assert key in r.stdout
