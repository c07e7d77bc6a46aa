"""The benchmark's command line on the CPU: more than one GPU is refused with a
message before anything touches a device, and every documented mode parses."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help_lists_every_mode():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workloads", "--col-slices", "--tile-shapes", "--small-systems",
                 "--pmc-probe", "--spmv-probe", "--no-cpu-baseline"):
        assert flag in r.stdout, flag
