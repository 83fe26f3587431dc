"""Host checks of the benchmark's command line (no GPU): more than one GPU is
refused with a message, and the help text lists the workloads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


def test_help_lists_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for cfg in ("C2", "C3", "C4", "C5"):
        assert cfg in r.stdout
