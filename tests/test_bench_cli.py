"""The benchmark script's command-line contract, checked without a GPU: one GPU only
(a request for more exits with a message before anything touches a device), and the
options a reader of the results needs to reproduce them."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True, timeout=120,
                       cwd=ROOT, env=env)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_help_lists_the_reproduction_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--operands", "--family", "--igemm-tile", "--calibrate-copy",
                "--pmc-summary", "--no-cpu-baseline", "--no-extras"):
        assert opt in r.stdout, opt
