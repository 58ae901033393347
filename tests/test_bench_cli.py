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
                 "--graph", "--no-side"):
        assert flag in r.stdout, flag


def test_cpu_baseline_sample_on_host():
    """The oracle leg of the bench on a small workload: a bounded sample,
    scaled to one step, with the cores of each leg stated."""
    sys.path.insert(0, ROOT)
    import numpy as np

    import bench
    from denoiser_attention_amd import synth
    cfg = synth.get_config("tiny_fp32").with_(batch=3)
    inp = synth.attn_inputs(cfg, seed=0)
    lg = synth.logits(cfg, seed=0)
    res = bench.cpu_baseline(cfg, inp, lg, np.ones((3, cfg.block_len), np.uint8), attn_seqs=2,
                             unmask_seqs=2)
    assert res["kind"] == "oracle" and res["unit"] == "block-tokens/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert res["cores_per_leg"]["unmask_processes"] == res["cores"]
    assert "scaled x1.5" in res["sample"]


def test_code_digest_ignores_comments_only():
    """The digest that ties counter-derived traffic to a kernel's source keeps
    its value across comment and layout edits and changes with any code."""
    sys.path.insert(0, ROOT)
    import bench

    a = "int f(int x) {  // twice\n  return 2 * x;\n}\n"
    b = "// doubles\nint f(int x) {    // two times x\n\n    return 2 * x;\n}\n"
    c = "int f(int x) {  // twice\n  return 3 * x;\n}\n"
    assert bench.code_digest(a) == bench.code_digest(b)
    assert bench.code_digest(a) != bench.code_digest(c)
    for kernel in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_digest(kernel)) == 16

