"""bench.py's command line on the host (no GPU): a request for more than one
GPU is refused with a message before anything touches a device, and the help
text lists the profiler workloads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n, "--steps", "1", "--warmup", "0")
        assert r.returncode == 2
        assert r.stdout == ""
        assert "one GPU only" in r.stderr and f"asked for {n}" in r.stderr


def test_help_lists_the_profiler_workloads():
    r = run("--help")
    assert r.returncode == 0
    for wl in ("decode", "prefill", "decode100b", "decode100b_1bit", "a48", "ffn", "pack", "copy"):
        assert wl in r.stdout
