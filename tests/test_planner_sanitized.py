"""The unit planner (plan.cpp, host C++) under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/host/plan_check.cpp applies the planned copy segments to host buffers for random units
of both layouts and checks every element against the layout definitions (each written
exactly once, from the right place), the per-parameter runs of each rank's shard, and that
oversized units are rejected as overflows."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "sharded_fsdp_flatten_amd", "csrc")
FLAGS = ["-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
         "-fno-sanitize-recover=undefined"]


def test_planner_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    probe = tmp_path / "probe.cpp"
    probe.write_text("int main() { return 0; }\n")
    if subprocess.run([gxx, *FLAGS, str(probe), "-o", str(tmp_path / "probe")],
                      capture_output=True).returncode != 0:
        pytest.skip("g++ has no sanitizer runtime here")
    exe = tmp_path / "plan_check"
    build = subprocess.run([gxx, *FLAGS, "-I", CSRC, os.path.join(ROOT, "tests", "host", "plan_check.cpp"),
                            os.path.join(CSRC, "plan.cpp"), "-o", str(exe)],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe), "400"], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "planner ok" in run.stdout
