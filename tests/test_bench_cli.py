"""CPU checks of bench.py's command line: more than one GPU is refused with a
message before anything touches a GPU, and so is a launch with WORLD_SIZE > 1
(as torch.distributed.run would start it)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_distributed_launch_is_refused():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
