"""Build the gfx950 attention library in-tree: ``libfa_mi355x.so`` next to this file.

Every source is compiled by hipcc for gfx950 only.  Packed fp32 VALU
instructions are disabled for the device code (-packed-fp32-ops); hipcc's host
pass warns that it does not know that feature, which is harmless.

    python -m exact_io_aware_30_amd.build [-v]
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_api.cpp"]
# Instruction-rate loops for the benchmark's measured ceilings: a library of
# their own, so that the attention library holds only the attention path.
RATES_SOURCES = ["fa_rates.hip"]
RATES_LIB_PATH = os.path.join(HERE, "libfa_rates.so")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA sources and accumulators in VGPRs: without this the backend keeps
    # accumulators in AGPRs and copies them through VGPRs for every VALU use.
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if "recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link both shared libraries; returns the
    attention library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = {}
    cmds = []
    for src in SOURCES + RATES_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs[src] = obj
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    for srcs, path in ((SOURCES, LIB_PATH), (RATES_SOURCES, RATES_LIB_PATH)):
        tmp = path + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(objs[s] for s in srcs), "-o", tmp], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
