"""bench.py command line checks that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT,
                           capture_output=True, text=True, timeout=120,
                           env={**os.environ, **env})
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""
