"""bench.py's command line, on the CPU: it measures one GPU and says so when
asked for more, and it rejects unknown legs, both before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_leg_is_rejected():
    r = _run("--legs", "backward,not_a_leg")
    assert r.returncode == 2
    assert "not_a_leg" in r.stderr
