"""Build libslm.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libslm.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # keep hipcc from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every .hip source into one shared library next to this file."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *HIP_FLAGS, "-I", os.path.join(HERE, "..", "include"), "-o", tmp, *sources()]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
