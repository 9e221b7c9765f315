"""bench.py's command line on the CPU: a request for more than one GPU exits
with status 2 and says why, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_multi_rank_launch_is_refused():
    r = _run("--gpus", "1", env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU only" in r.stderr
