"""bench.py's command-line contract on the host: runs it cannot measure are
refused with exit status 2 and a message, before any GPU work."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    env = dict(os.environ, WORLD_SIZE="1")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("extra", [(), ("--only", "decode"), ("--only", "verify")])
def test_zero_inputs_needs_a_prefill_entry(extra):
    r = _bench("--zero-inputs", *extra)
    assert r.returncode == 2
    assert "--zero-inputs needs --only prefill" in r.stderr
    assert r.stdout == ""
