"""Compile liblcmp.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "liblcmp.so")
ARCH = os.environ.get("LCMP_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(force: bool = False, verbose: bool = False) -> str:
    """Build liblcmp.so unless it is present and newer than every source."""
    srcs = sources()
    hdrs = glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(HERE, "..", "include", "lcmp.h")]
    if not force and os.path.exists(SO):
        newest = max(os.path.getmtime(f) for f in srcs + hdrs)
        if os.path.getmtime(SO) >= newest:
            return SO
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = SO + ".tmp"
    cmd = [hipcc, *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(force=True, verbose=True))
