"""bench.py on more than one GPU: it measures one GPU only and says so,
before it touches a device."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.mark.parametrize("argv, world", [(["--gpus", "2"], "1"), (["--gpus", "8"], "1"),
                                         ([], "2")])
def test_more_than_one_gpu_exits_with_a_message(argv, world):
    env = dict(os.environ, WORLD_SIZE=world)
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), *argv], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_unknown_config_is_refused_before_the_gpu():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--config", "no_such_shape"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "no workload 'no_such_shape'" in r.stderr
    assert r.stdout == ""
