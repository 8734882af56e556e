"""The boundary is a C ABI: include/fsdp_flatten.h must compile as strict C99 and a C program
must link libfsdpflat.so and call it.  tests/host/abi_c_check.c is built with gcc
(-std=c99 -pedantic -Werror) and run; it exercises the host-side calls (unit sizes fixed by the
layout definitions for hand-worked units) and error statuses (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "host", "abi_c_check.c")
LIBDIR = os.path.join(ROOT, "sharded_fsdp_flatten_amd")


def test_header_is_c99_and_the_library_links_from_c(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    if not os.path.exists(os.path.join(LIBDIR, "libfsdpflat.so")):
        raise RuntimeError("libfsdpflat.so is not built; run __graft_entry__.build()")
    exe = str(tmp_path / "abi_c_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), SRC, "-L", LIBDIR, "-lfsdpflat",
           "-Wl,-rpath," + LIBDIR, "-o", exe]
    c = subprocess.run(cmd, capture_output=True, text=True)
    assert c.returncode == 0, c.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.gpu
def test_data_path_driven_from_c_matches_the_oracle(tmp_path):
    """tests/host/abi_c_gpu.c: hipMalloc'd buffers, every call through the C header (flatten of
    all ranks and of one rank of a padded unit, copy-out, AdamW twice, a 5-rank reduction and a
    32-rank one long enough for the row-major sweep), compared bit for bit with the oracle's C
    functions; no Python or torch on the data path."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    oracle_dir = os.path.join(ROOT, "oracle")
    for lib in (os.path.join(LIBDIR, "libfsdpflat.so"), os.path.join(oracle_dir, "liboracle.so")):
        if not os.path.exists(lib):
            raise RuntimeError("%s is not built; run __graft_entry__.build()" % lib)
    exe = str(tmp_path / "abi_c_gpu")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(rocm, "include"),
           os.path.join(ROOT, "tests", "host", "abi_c_gpu.c"),
           "-L", LIBDIR, "-lfsdpflat", "-L", oracle_dir, "-loracle",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + ":".join([LIBDIR, oracle_dir, os.path.join(rocm, "lib")]), "-o", exe]
    c = subprocess.run(cmd, capture_output=True, text=True)
    assert c.returncode == 0, c.stderr
    print("running %s" % exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
