"""bench.py's command line on a host without a GPU: a request for several
GPUs is refused with a message, before any device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_several_gpus_refused_with_message():
    p = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout.strip() == ""


def test_world_size_above_one_refused():
    p = run_bench("--steps", "1", env_extra={"WORLD_SIZE": "4"})
    assert p.returncode == 2
    assert "one GPU" in p.stderr
