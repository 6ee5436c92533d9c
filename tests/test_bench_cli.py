"""Host-only checks of the benchmark's command line (no GPU needed)."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_a_distributed_launch():
    env = {"WORLD_SIZE": "4", "PATH": "/usr/bin:/bin"}
    r = subprocess.run([sys.executable, str(ROOT / "bench.py")], capture_output=True, text=True, timeout=120,
                       env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
