"""Build libfsdpflat.so (the C-ABI library) in-tree with hipcc for gfx950, and
libfsdpprobe.so (hardware floor probes the benchmark times beside the library;
not part of the data path).

    python -m sharded_fsdp_flatten_amd.build

Flags that matter for results:
  -ffp-contract=off        every float operation rounds on its own (no FMA),
                           matching the CPU oracle's operation order;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                           no packed-fp32 instructions are generated;
  no -ffast-math / -fgpu-flush-denormals-to-zero: IEEE division, square root
                           and subnormals.
A flag that matters for speed only:
  -mllvm -amdgpu-kernarg-preload-count=16
                           the first 16 dwords of a kernel's scalar arguments
                           arrive preloaded in scalar registers (the copy engine,
                           AdamW and the sums of squares pass what a workgroup
                           needs first that way), so a short-lived workgroup
                           issues its loads without waiting for a scalar load.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfsdpflat.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["kernels.hip", "plan.cpp", "fsdp_abi.cpp"]
PROBE_LIB_PATH = os.path.join(HERE, "libfsdpprobe.so")
PROBE_SOURCES = ["probes.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]


def _link(sources, path, verbose):
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout)
        raise RuntimeError("hipcc failed to build %s" % os.path.basename(path))
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    _link(SOURCES, LIB_PATH, verbose)
    _link(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
