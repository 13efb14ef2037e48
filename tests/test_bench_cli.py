"""bench.py's command-line contract on a machine without a GPU: more than one GPU
is refused with a message, and without a device it exits non-zero instead of
printing a result line."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    env = dict(os.environ, CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def test_no_device_prints_no_result():
    r = run_bench("--steps", "1", "--warmup", "0", "--no-cpu")
    assert r.returncode != 0
    assert not any(line.startswith("{") for line in r.stdout.splitlines())
