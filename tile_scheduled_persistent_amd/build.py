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
# The worker units each instantiate the persistent worker for one weight format, token selection
# and KV format, or (the _mt units) the multi-token verify workers of one weight format (they
# include kernel.hip); every source compiles to an object of its own, in parallel, then links.
WORKER_UNITS = [f"workers_{w}{s}{k}.hip" for w in ("bf16", "int8") for s in ("", "_sampled") for k in ("", "_kv8")] + [
    "workers_bf16_mt.hip", "workers_int8_mt.hip", "workers_bf16_mt_kv8.hip", "workers_int8_mt_kv8.hip"]
SOURCES = ["kernel.hip", *WORKER_UNITS, "planner.cpp", "api.cpp"]
HEADERS = ["plan_types.h", "planner.h"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# CDNA4 code generation flags: packed-FP32 instructions are disabled everywhere.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-unit scheduling: the worker units use the backend's iterative ILP scheduler (measured faster:
# +1.4 % on the Llama-3.2-1B shape, +3 % sampled and at 32K positions, +1.2 % INT8 weights), except
# those with the INT8 KV cache, which were 1.5 % faster with the default scheduler.
ILP_SCHED = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]


def unit_flags(src: str) -> list:
    return ILP_SCHED if src.startswith("workers_") and "_kv8" not in src else []


def build_id() -> str:
    """64-bit id of the worker binary: hash of every source and header and of the flags each source
    is compiled with."""
    h = hashlib.sha256()
    h.update(" ".join(DEVICE_FLAGS).encode())
    for name in SOURCES + HEADERS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(" ".join(unit_flags(name)).encode())
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "tiles.h"), "rb") as f:
        h.update(f.read())
    return "0x" + h.hexdigest()[:16] + "ull"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[-3:])}\n{errs}")
    if verbose and errs:
        print(errs, file=sys.stderr)


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor

    bid = build_id()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [HIPCC, "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", *DEVICE_FLAGS,
              f"-DTILES_BUILD_ID={bid}", "-I", os.path.join(ROOT, "include")]
    objs = [os.path.join(objdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, common + unit_flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
                for src, obj in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
