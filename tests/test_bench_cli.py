"""bench.py's command line on the CPU: more than one GPU is refused with a
message and exit status 2, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = run_bench(["--steps", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr
