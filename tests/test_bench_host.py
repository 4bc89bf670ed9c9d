"""bench.py's one-GPU contract, on the CPU: asked for more than one GPU (by flag
or by a launcher's WORLD_SIZE) it exits with status 2 and says why, before
touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_by_flag_exits_2():
    res = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert res.returncode == 2
    assert "one GPU only" in res.stderr and res.stdout == ""


def test_more_than_one_rank_by_world_size_exits_2():
    res = _run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert res.returncode == 2
    assert "WORLD_SIZE=4" in res.stderr and res.stdout == ""
