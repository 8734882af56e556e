"""bench.py's command line, checked without a GPU."""
import os
import subprocess
import sys

from conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    for n in ("2", "8"):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], cwd=ROOT,
                           stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=60)
        assert p.returncode == 2
        assert "ONE GPU" in p.stderr and p.stdout == ""
