"""The bench's command-line contract that needs no GPU: more than one GPU is
refused with a message and a non-zero status before anything touches a
device, and the help text lists every timed section."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_sections():
    r = run("--help")
    assert r.returncode == 0
    for name in ("step", "step_sweep", "infer", "serve", "serve_sweep", "conv", "layer", "routes", "copy"):
        assert name in r.stdout
