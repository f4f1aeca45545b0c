"""Build ``libtiles.so`` (HIP kernel + host planner/runtime) for gfx950 in-tree.

Run as ``python -m tile_scheduled_persistent_amd.build``.  hipcc cross-compiles the
device code, so this works on a machine without a GPU.
"""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtiles.so")
SOURCES = ["kernel.hip", "planner.cpp", "api.cpp"]
HEADERS = ["plan_types.h", "planner.h"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# CDNA4 code generation flags: packed-FP32 instructions are disabled everywhere.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_id() -> str:
    """64-bit id of the worker binary: hash of every source and header."""
    h = hashlib.sha256()
    for name in SOURCES + HEADERS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "tiles.h"), "rb") as f:
        h.update(f.read())
    return "0x" + h.hexdigest()[:16] + "ull"


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", *DEVICE_FLAGS,
           f"-DTILES_BUILD_ID={build_id()}", "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs:
        print(errs, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
