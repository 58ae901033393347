"""bench.py's command line on the host: a request for more than one GPU exits
with a message and status 2, and the measurement modes are all offered.
Nothing here touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
    assert "{" not in r.stdout   # no JSON line


def test_help_lists_every_mode():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--config", "--suite", "--attn-only",
                 "--lmhead-only", "--kernel-reps", "--copy-calibration", "--no-cpu-baseline",
                 "--graph"):
        assert flag in r.stdout, flag
