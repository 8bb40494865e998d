"""Host-side checks of bench.py's contract (no GPU): more than one GPU is refused with a
message before any device work, and the command line parses."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_command_line_parses():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--backward", "--ep-shards", "--tiled"):
        assert opt in r.stdout
