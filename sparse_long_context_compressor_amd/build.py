"""Build libslc.so (the C-ABI HIP library) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libslc.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # gfx950: keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
