"""bench.py's command line without a GPU: more than one GPU is refused with
a message, and the help text lists the documented flags."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    res = _run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_help_lists_flags():
    res = _run("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--graph", "--no-cpu-baseline",
                 "--batch-requests", "--copy-probe"):
        assert flag in res.stdout, flag
