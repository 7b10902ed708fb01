"""bench.py's refusal of several GPUs: the library runs on one MI355X, so any
request for more than one GPU (the --gpus flag or a WORLD_SIZE from a
launcher) ends with status 2 and a message on stderr, before the GPU or the
oracle is touched, and no result line is printed."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None),
                                      (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(args, env):
    p = _run(args, env)
    assert p.returncode == 2, (p.returncode, p.stderr[-500:])
    assert "measures one GPU only" in p.stderr
    assert p.stdout.strip() == ""
