"""Build libsparse_decode.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_decode.so")
SOURCES = ["sd_kernels.hip", "sd_runtime.hip", "sd_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


LIB_TIMELINE = os.path.join(HERE, "libsparse_decode_timeline.so")


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile the library; timeline=True builds the measurement variant
    (per-phase timestamps of the one-launch step, SD_TIMELINE) instead."""
    out = LIB_TIMELINE if timeline else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ([HIPCC] + FLAGS + (["-DSD_TIMELINE"] if timeline else []) +
           [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
    sys.exit(0)
